"""Decode with a fused KV-cache append (GPU): parity with the oracle (append,
then attend), the caches after the call bit for bit, and the result bit for
bit equal to a plain decode over the caches the oracle updated.  The
generator leaves NaN in the current tokens' slots, standing for cache memory
not yet written, so a kernel that read a stale slot would fail parity."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from gpu_util import bits_of, dev_bf16, dev_i32, host_f64, need_gpu
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_append(p: gen.DecodeAppend, rounding="rtne"):
    d = p.base
    kc, vc = dev_bf16(d.k_pool), dev_bf16(d.v_pool)
    o, lse = ea.attn_decode_paged_append(dev_bf16(d.q), dev_bf16(p.k_new), dev_bf16(p.v_new),
                                         kc, vc, dev_i32(d.block_table), dev_i32(d.seq_lens),
                                         scale=d.scale, rounding=rounding)
    torch.cuda.synchronize()
    return o, lse, kc, vc


def check_append(p: gen.DecodeAppend, o, lse, kc, vc, what=""):
    d = p.base
    o_ref, l_ref, kp, vp = att.decode_paged_append(d.q, p.k_new, p.v_new, d.k_pool, d.v_pool,
                                                   d.block_table, d.seq_lens, d.Hkv, d.scale)
    check_o(host_f64(o), o_ref, what)
    check_lse(host_f64(lse), l_ref, what)
    # caches: bit for bit (NaN slots compare as bit patterns)
    assert np.array_equal(bits_of(kc), kp), f"{what}: K cache"
    assert np.array_equal(bits_of(vc), vp), f"{what}: V cache"
    return kp, vp


CASES = [
    # B, Hq, Hkv, max_len, lens
    (1, 1, 1, 16, [1]),                    # the only token is the new one
    (3, 4, 1, 64, [1, 16, 17]),            # new token first / last in its page
    (4, 8, 8, 300, [300, 1, 129, 32]),
    (5, 32, 8, 1000, None),
    (2, 32, 1, 700, [700, 513]),           # MQA
    (2, 40, 2, 500, [499, 100]),           # two head blocks per K/V head: one writer
    (130, 4, 1, 100, None),                # many sequences, chunks across them
    (2, 16, 2, 20000, [20000, 3001]),      # many parts per sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_L{c[3]}")
def test_append_parity_and_caches(case):
    B, Hq, Hkv, L, lens = case
    p = gen.decode_append_inputs(B, Hq, Hkv, max_len=L, seed=B * 13 + L, lens=lens)
    o, lse, kc, vc = run_append(p)
    kp, vp = check_append(p, o, lse, kc, vc, str(case))
    # the same kernels over the caches the oracle updated, without the append
    d = p.base
    o2, l2 = ea.attn_decode_paged(dev_bf16(d.q), dev_bf16(kp), dev_bf16(vp),
                                  dev_i32(d.block_table), dev_i32(d.seq_lens), scale=d.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "append != write + decode"
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))


def test_append_config5_and_repeat():
    """The decode workload with an append; a second call on the updated
    caches (the same rows written again) gives the same bits."""
    p = gen.decode_append_inputs(32, 32, 8, max_len=4096, seed=5)
    d = p.base
    kc, vc = dev_bf16(d.k_pool), dev_bf16(d.v_pool)
    args = (dev_bf16(d.q), dev_bf16(p.k_new), dev_bf16(p.v_new), kc, vc, dev_i32(d.block_table),
            dev_i32(d.seq_lens))
    o1, l1 = ea.attn_decode_paged_append(*args, scale=d.scale)
    torch.cuda.synchronize()
    check_append(p, o1, l1, kc, vc, "config5 append")
    o2, l2 = ea.attn_decode_paged_append(*args, scale=d.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_append_with_rounding_rules():
    p = gen.decode_append_inputs(6, 24, 2, max_len=900, seed=41)
    res = {}
    for mode in ("rtne", "rtna", "rtz"):
        o, lse, kc, vc = run_append(p, mode)
        check_append(p, o, lse, kc, vc, mode)
        res[mode] = bits_of(o).astype(np.int32)
    assert np.all((res["rtne"] - res["rtz"] >= 0) & (res["rtne"] - res["rtz"] <= 1))
    assert np.all((res["rtna"] - res["rtz"] >= 0) & (res["rtna"] - res["rtz"] <= 1))


def test_append_to_an_out_of_range_page_writes_nothing():
    """A table entry outside [0, num_pages) for the current token's page is
    out of contract: nothing is written and that page's tokens are left out
    (as the plain decode does)."""
    p = gen.decode_append_inputs(3, 8, 2, max_len=100, seed=43, lens=[40, 17, 100])
    d = p.base
    tab = d.block_table.copy()
    tab[1, 1] = d.num_pages + 3            # page of token 16 of sequence 1
    kc, vc = dev_bf16(d.k_pool), dev_bf16(d.v_pool)
    o, lse = ea.attn_decode_paged_append(dev_bf16(d.q), dev_bf16(p.k_new), dev_bf16(p.v_new),
                                         kc, vc, dev_i32(tab), dev_i32(d.seq_lens),
                                         scale=d.scale)
    torch.cuda.synchronize()
    _, _, kp, vp = att.decode_paged_append(d.q, p.k_new, p.v_new, d.k_pool, d.v_pool,
                                           d.block_table, d.seq_lens, d.Hkv, d.scale)
    # sequence 1's slot is untouched; the others are written
    pg, sl = d.block_table[1, 1], 0
    kp[pg, sl] = d.k_pool[pg, sl]
    vp[pg, sl] = d.v_pool[pg, sl]
    assert np.array_equal(bits_of(kc), kp) and np.array_equal(bits_of(vc), vp)
    # sequences 0 and 2 as the oracle; sequence 1 attends to its first page only
    o_ref, l_ref, _, _ = att.decode_paged_append(d.q, p.k_new, p.v_new, d.k_pool, d.v_pool,
                                                 d.block_table, d.seq_lens, d.Hkv, d.scale)
    for b in (0, 2):
        check_o(host_f64(o[b]), o_ref[b], f"seq {b}")
        check_lse(host_f64(lse[b]), l_ref[b], f"seq {b}")
    one = gen.Decode(d.q[1:2], d.k_pool, d.v_pool, d.block_table[1:2], np.array([16], np.int32),
                     1, d.Hq, d.Hkv, d.scale)
    o1, l1 = att.decode_paged(one.q, one.k_pool, one.v_pool, one.block_table, one.seq_lens,
                              one.Hkv, one.scale)
    check_o(host_f64(o[1]), o1[0], "seq 1")
    check_lse(host_f64(lse[1]), l1[0], "seq 1")


def test_append_argument_errors():
    p = gen.decode_append_inputs(2, 8, 2, max_len=64, seed=44)
    d = p.base
    with pytest.raises(ValueError):
        ea.attn_decode_paged_append(dev_bf16(d.q), dev_bf16(p.k_new[:, :1]), dev_bf16(p.v_new),
                                    dev_bf16(d.k_pool), dev_bf16(d.v_pool),
                                    dev_i32(d.block_table), dev_i32(d.seq_lens))
