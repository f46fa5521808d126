"""The three rounding rules of the bf16 output (GPU).

Exact checks: with every key of a (sequence, K/V head) equal, every visible
probability is exactly 1 and O is the plain mean of the visible V rows; with V
values of few significant bits and a power-of-two number of visible keys that
mean is exact in float32, so the bf16 result of each rule is fixed bit for bit
(the closed form of identical keys, rounded by oracle.rounding).  Ties, where
RTNE and RTNA part, make up a large share of these outputs.

General checks, on random inputs: each rule within the parity tolerance of the
oracle, and the three results consistent with coming from the same float32
value (RTZ is the truncation; RTNE and RTNA add at most one unit to its
magnitude and differ only on ties); LSE independent of the rule; the rounded
entry points with RTNE equal the plain ones bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
import oracle.rounding as rnd
from gpu_util import bits_of, dev_bf16, dev_i32, host_f64, logical_o, need_gpu
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu

MODES = ("rtne", "rtna", "rtz")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def fwd(p: gen.Prefill, mode: str):
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    o, lse = ea.attn_fwd(q, k, v, causal=p.causal, scale=p.scale, rounding=mode,
                         layout="bshd" if p.layout == gen.BSHD else "bhsd")
    torch.cuda.synchronize()
    return o, lse


def dec(d: gen.Decode, mode: str):
    o, lse = ea.attn_decode_paged(dev_bf16(d.q), dev_bf16(d.k_pool), dev_bf16(d.v_pool),
                                  dev_i32(d.block_table), dev_i32(d.seq_lens), scale=d.scale,
                                  rounding=mode)
    torch.cuda.synchronize()
    return o, lse


def logical_bits(o: torch.Tensor, layout: int) -> np.ndarray:
    b = bits_of(o)
    return b.transpose(0, 2, 1, 3) if layout == gen.BSHD else b


def logical_v(p: gen.Prefill) -> np.ndarray:
    """V as float64 [B, Hkv, Sk, D]."""
    v = att.bf16_to_f64(p.v)
    return v.transpose(0, 2, 1, 3) if p.layout == gen.BSHD else v


def exact_sum_bound_ok(vals: np.ndarray, binades: int) -> bool:
    """Every partial sum of these values is exact in float32: they are
    multiples of 2^(-7-binades) and their magnitudes add up to below
    2^(24-7-binades)."""
    return float(np.abs(vals).sum(axis=-2).max()) < 2.0 ** (17 - binades)


EXACT_PREFILL = [
    # B, Hq, Hkv, Sq, Sk, layout, causal, binades
    (1, 4, 2, 300, 2, gen.BSHD, False, 0),     # about half the outputs are ties
    (1, 2, 2, 40, 2, gen.BHSD, False, 6),      # values over 13 binades
    (2, 2, 1, 257, 4, gen.BHSD, False, 5),
    (1, 2, 2, 64, 64, gen.BSHD, False, 2),
    (1, 2, 1, 520, 512, gen.BHSD, False, 0),   # 8 key tiles, ragged query tail
    (1, 4, 2, 256, 256, gen.BSHD, True, 0),    # causal: rows with 2^k visible keys
]


@pytest.mark.parametrize("case", EXACT_PREFILL, ids=lambda c: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "bshd" if c[5] == 0 else "bhsd", "causal" if c[6] else "full"))
def test_prefill_rules_bit_exact_on_exact_means(case):
    B, Hq, Hkv, Sq, Sk, lay, causal, binades = case
    p = gen.equal_keys_prefill(B, Hq, Hkv, Sq, Sk, layout=lay, causal=causal, seed=Sq + Sk,
                               binades=binades)
    v = logical_v(p)                                           # [B, Hkv, Sk, D]
    assert exact_sum_bound_ok(v, binades)
    G = Hq // Hkv
    # visible keys per query row (bottom-right causal alignment)
    i = np.arange(Sq)
    nvis = np.minimum(Sk, np.maximum(0, i + 1 + (Sk - Sq))) if causal else np.full(Sq, Sk)
    exact_rows = (nvis > 0) & ((nvis & (nvis - 1)) == 0)       # power-of-two counts
    assert exact_rows.sum() >= min(Sq, 8)
    csum = np.cumsum(v, axis=2)                                # exact: short values
    mean = np.empty((B, Hq, Sq, 128))
    for h in range(Hq):
        c = csum[:, h // G]                                    # [B, Sk, D]
        mean[:, h] = c[:, np.maximum(nvis - 1, 0)] / np.maximum(nvis, 1)[None, :, None]
    # the oracle agrees with the closed form of identical keys
    o_ref, _ = att.attention(p.q, p.k, p.v, B, Hq, Hkv, Sq, Sk, p.scale, causal, p.layout)
    assert np.allclose(o_ref, mean, rtol=1e-13, atol=1e-13)
    for mode in MODES:
        o, _ = fwd(p, mode)
        got = logical_bits(o, lay)[:, :, exact_rows]
        want = rnd.bf16_bits(rnd.round_bf16(mean[:, :, exact_rows], mode))
        bad = np.argwhere(got != want)
        assert bad.size == 0, (mode, bad[:4].tolist(), [hex(got[tuple(x)]) for x in bad[:4]],
                               [hex(want[tuple(x)]) for x in bad[:4]])
        if not exact_rows.all():                               # other rows: parity tolerance
            check_o(logical_o(o, lay)[:, :, ~exact_rows], o_ref[:, :, ~exact_rows], mode)
    if Sk <= 4 and binades == 0:                               # the ties are exercised
        ne = rnd.round_bf16(mean[:, :, exact_rows], "rtne")
        na = rnd.round_bf16(mean[:, :, exact_rows], "rtna")
        assert (ne != na).mean() > 0.1


def test_decode_rules_bit_exact_on_single_part_sequences():
    """Sequences laid out so that each one falls in a single chunk of four
    pages (11 sequences, 16 pages), so the merge passes one exact mean on."""
    lens = [64, 32, 32, 16, 16, 16, 16, 8, 4, 2, 1]
    d = gen.equal_keys_decode(lens, 8, 2, seed=11, binades=3)
    G = d.Hq // d.Hkv
    vb = att.bf16_to_f64(d.v_pool)
    mean = np.empty((d.B, d.Hq, 128))
    for b, n in enumerate(lens):
        rows = np.stack([vb[d.block_table[b, t // 16], t % 16] for t in range(n)])  # [n, Hkv, D]
        assert exact_sum_bound_ok(rows.transpose(1, 0, 2), 3)
        m = rows.sum(axis=0) / n
        for h in range(d.Hq):
            mean[b, h] = m[h // G]
    o_ref, _ = att.decode_paged(d.q, d.k_pool, d.v_pool, d.block_table, d.seq_lens, d.Hkv,
                                d.scale)
    assert np.allclose(o_ref, mean, rtol=1e-13, atol=1e-13)
    for mode in MODES:
        o, _ = dec(d, mode)
        got = bits_of(o)
        want = rnd.bf16_bits(rnd.round_bf16(mean, mode))
        bad = np.argwhere(got != want)
        assert bad.size == 0, (mode, bad[:4].tolist())


def check_same_source(res: dict):
    """RTNE, RTNA and RTZ bit patterns consistent with rounding one float32
    value: RTZ is the truncation t; RTNE and RTNA are t or t + 1 (one unit more
    magnitude, i.e. bit pattern + 1 for either sign); where they differ it is a
    tie, RTNE = t with an even last bit and RTNA = t + 1."""
    t = res["rtz"].astype(np.int32)
    ne = res["rtne"].astype(np.int32)
    na = res["rtna"].astype(np.int32)
    assert np.all((ne == t) | (ne == t + 1))
    assert np.all((na == t) | (na == t + 1))
    assert np.all(na >= ne)
    diff = ne != na
    assert np.all(ne[diff] == t[diff]) and np.all((t[diff] & 1) == 0)


CONSISTENCY = [
    (1, 4, 2, 300, 333, gen.BSHD, False),
    (2, 4, 1, 257, 257, gen.BHSD, True),
    (1, 2, 2, 100, 700, gen.BHSD, True),
    (2, 16, 16, 2100, 200, gen.BSHD, False),   # 288 workgroups, ragged last query tile
]


@pytest.mark.parametrize("case", CONSISTENCY, ids=lambda c: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d" % c[:5])
def test_prefill_rules_parity_and_consistency(case):
    B, Hq, Hkv, Sq, Sk, lay, causal = case
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=lay, causal=causal, seed=Sq * 3 + Sk,
                           n_hot=4)
    o_ref, l_ref = att.attention(p.q, p.k, p.v, B, Hq, Hkv, Sq, Sk, p.scale, causal, p.layout)
    res, lses = {}, {}
    for mode in MODES:
        o, lse = fwd(p, mode)
        check_o(logical_o(o, lay), o_ref, mode)
        check_lse(host_f64(lse), l_ref, mode)
        res[mode] = bits_of(o)
        lses[mode] = lse.cpu().numpy().view(np.uint32)
    check_same_source(res)
    assert np.array_equal(lses["rtne"], lses["rtna"]) and np.array_equal(lses["rtne"], lses["rtz"])
    assert (res["rtne"] != res["rtz"]).mean() > 0.3            # the rules do differ


def test_decode_rules_parity_and_consistency():
    d = gen.decode_inputs(5, 32, 8, max_len=1000, seed=21)
    o_ref, l_ref = att.decode_paged(d.q, d.k_pool, d.v_pool, d.block_table, d.seq_lens, d.Hkv,
                                    d.scale)
    res, lses = {}, {}
    for mode in MODES:
        o, lse = dec(d, mode)
        check_o(host_f64(o), o_ref, mode)
        check_lse(host_f64(lse), l_ref, mode)
        res[mode] = bits_of(o)
        lses[mode] = lse.cpu().numpy().view(np.uint32)
    check_same_source(res)
    assert np.array_equal(lses["rtne"], lses["rtna"]) and np.array_equal(lses["rtne"], lses["rtz"])


def test_rounded_entry_points_with_rtne_equal_the_plain_ones():
    p = gen.prefill_inputs(1, 4, 2, 300, 333, layout=gen.BSHD, seed=5)
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    o1, l1 = ea.attn_fwd(q, k, v, scale=p.scale)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    st = ea.library().attn_fwd_rounded(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), 1, 4, 2, 300, 333,
        128, ctypes.c_float(p.scale), 0, gen.BSHD, ea.ROUNDING["rtne"],
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))

    d = gen.decode_inputs(3, 8, 2, max_len=300, seed=6)
    a1 = dec(d, "rtne")
    qd, kd, vd = dev_bf16(d.q), dev_bf16(d.k_pool), dev_bf16(d.v_pool)
    tab, lens = dev_i32(d.block_table), dev_i32(d.seq_lens)
    need = ea.attn_decode_workspace_bytes(d.B, d.Hq, d.max_blocks)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o3 = torch.empty_like(qd)
    l3 = torch.empty((d.B, d.Hq), dtype=torch.float32, device="cuda")
    st = ea.library().attn_decode_paged_rounded(
        qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), tab.data_ptr(), lens.data_ptr(),
        o3.data_ptr(), l3.data_ptr(), d.B, d.Hq, d.Hkv, 128, 16, d.max_blocks, d.num_pages,
        ctypes.c_float(d.scale), ea.ROUNDING["rtne"], ws.data_ptr(), need,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(a1[0].view(torch.int16), o3.view(torch.int16))
    assert torch.equal(a1[1].view(torch.int32), l3.view(torch.int32))
