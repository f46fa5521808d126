"""Seeded generator and tolerance helper (CPU only)."""
import math

import numpy as np
import torch

import attn_inputs as gen
from tolerance import ulp_bf16, o_tolerance


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.4e38, 1e-40],
                                 np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_tie_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert gen.f32_to_bf16_bits(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert gen.f32_to_bf16_bits(np.float32(1 + 3 * 2 ** -8)) == 0x3F82


def test_generator_is_deterministic_and_seeded():
    a = gen.prefill_inputs(1, 2, 1, 33, 17, seed=5, n_hot=3)
    b = gen.prefill_inputs(1, 2, 1, 33, 17, seed=5, n_hot=3)
    c = gen.prefill_inputs(1, 2, 1, 33, 17, seed=6, n_hot=3)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    assert a.hot_rows == b.hot_rows and len(a.hot_rows) == 3


def test_hot_rows_are_scaled_by_8():
    base = gen.prefill_inputs(1, 4, 4, 256, 256, seed=1)
    hot = gen.config1()
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    diff = np.argwhere(np.any(base.q != hot.q, axis=-1))
    assert sorted(map(tuple, diff.tolist())) == sorted(hot.hot_rows)
    for (b, s, h) in hot.hot_rows:
        assert np.array_equal(f(hot.q[b, s, h]), 8 * f(base.q[b, s, h]))


def test_distributions():
    p = gen.prefill_inputs(1, 4, 4, 2048, 2048, seed=9, v_dist="uniform")
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, v = f(p.q), f(p.v)
    assert abs(q.mean()) < 0.01 and abs(q.std() - 1) < 0.01
    assert v.min() >= -1 and v.max() <= 1 and abs(v.std() - 1 / math.sqrt(3)) < 0.01


def test_decode_structure():
    d = gen.decode_inputs(32, 32, 8, max_len=4096, seed=5)
    assert d.block_table.dtype == np.int32 and d.block_table.shape == (32, 256)
    nb = (d.seq_lens + 15) // 16
    ids = np.concatenate([d.block_table[b, :nb[b]] for b in range(32)])
    assert np.array_equal(np.sort(ids), np.arange(d.num_pages))  # a permutation
    assert not np.array_equal(ids, np.arange(d.num_pages))
    for b in range(32):
        assert np.all(d.block_table[b, nb[b]:] == -1)
        t = int(d.seq_lens[b]) % 16
        last = d.block_table[b, nb[b] - 1]
        if t:
            assert np.all(d.k_pool[last, t:] == 0x7FC0) and np.all(d.v_pool[last, t:] == 0x7FC0)
        assert not np.any(d.k_pool[last, :t if t else 16] == 0x7FC0)
    assert 1 <= d.seq_lens.min() and d.seq_lens.max() <= 4096
    assert d.bytes > 4096 * d.tokens


def test_ulp_bf16():
    x = np.array([1.0, 1.5, 0.75, 2.0, 0.0, 2.0 ** -130, -3.0, 255.0, 256.0])
    want = np.array([2 ** -7, 2 ** -7, 2 ** -8, 2 ** -6, 2 ** -133, 2 ** -133, 2 ** -6,
                     1.0, 2.0])
    assert np.array_equal(ulp_bf16(x), want)
    assert np.allclose(o_tolerance(np.array([1.0, 0.0])), [2 * 2 ** -7 + 1e-3, 1e-3])
