"""The forward with prepared fp16 V^T tiles (attn_prep_v + attn_fwd_prepped)
against the single-call forward (attn_fwd / attn_fwd_rounded) on the same
inputs: both round V and P to fp16 and run the same products in the same
order, so O and LSE must agree bit for bit (GPU).  Parity of either with the
fp64 oracle is covered by the other forward tests: through the binding's
default, the full-size workloads run the prepared path and the smaller
shapes the single call."""

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
from gpu_util import bits_of, dev_bf16, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def both(p, rounding="rtne", q2=None):
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    d = p.q.shape[-1]
    lay = "bshd" if p.layout == gen.BSHD else "bhsd"
    kw = dict(causal=p.causal, scale=p.scale, layout=lay, rounding=rounding)
    o1, l1 = ea.attn_fwd(q, k, v, prepare_v=False, **kw)
    nvt = ea.attn_prep_v_bytes(p.B, p.Hq, p.Hkv, p.Sk, d)
    assert nvt > 0
    vt = torch.full((nvt,), 0x7f, dtype=torch.uint8, device=q.device)
    o2, l2 = ea.attn_fwd(q, k, v, vt=vt, prepare_v=True, **kw)
    torch.cuda.synchronize()
    print(f"case: B{p.B} Hq{p.Hq} Hkv{p.Hkv} Sq{p.Sq} Sk{p.Sk} d{d} {lay} causal={p.causal} "
          f"{rounding}", flush=True)
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32))
    return q, k, v, vt, kw


SHAPES = [
    # B, Hq, Hkv, Sq, Sk, layout, causal: groups of 1, 2, 3 (prefill kernel,
    # 64-key tiles) and of 4k (GQA kernel, 32-key tiles)
    (1, 2, 2, 1, 1, gen.BSHD, False),
    (1, 2, 1, 17, 15, gen.BSHD, False),
    (2, 4, 2, 63, 65, gen.BHSD, False),
    (1, 3, 3, 129, 127, gen.BSHD, True),
    (1, 6, 2, 300, 300, gen.BSHD, True),
    (2, 4, 4, 257, 257, gen.BHSD, True),
    (1, 4, 4, 513, 200, gen.BSHD, False),
    (1, 2, 2, 100, 700, gen.BHSD, True),
    (1, 2, 1, 400, 150, gen.BSHD, True),
    (3, 2, 2, 1, 333, gen.BHSD, True),
    (2, 8, 8, 1024, 1024, gen.BHSD, False),   # 64 workgroups of 16 tiles
    (1, 16, 16, 600, 2000, gen.BSHD, True),   # 48 workgroups, ragged tails
    (1, 4, 1, 1, 1, gen.BSHD, False),
    (1, 4, 1, 33, 31, gen.BSHD, False),
    (2, 8, 2, 100, 97, gen.BHSD, True),
    (1, 8, 1, 300, 700, gen.BSHD, True),
    (1, 16, 2, 257, 129, gen.BHSD, False),
    (2, 32, 8, 500, 1000, gen.BSHD, True),    # cfg3's group shape, ragged
    (1, 4, 1, 400, 150, gen.BSHD, True),      # Sq > Sk: first rows see no key
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s" % (
    s[0], s[1], s[2], s[3], s[4], "bshd" if s[5] == 0 else "bhsd", "causal" if s[6] else "full"))
def test_prepped_equals_single_call(shape):
    B, Hq, Hkv, Sq, Sk, layout, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=11 + Sq + Sk)
    both(p)


SHAPES_D256 = [
    # head dim 256: 32-key tiles, 128 query rows per workgroup
    (1, 2, 2, 1, 1, gen.BSHD, False),
    (1, 2, 1, 17, 15, gen.BSHD, False),
    (2, 4, 2, 63, 65, gen.BHSD, False),
    (1, 3, 3, 129, 127, gen.BSHD, True),
    (1, 4, 4, 257, 257, gen.BHSD, True),
    (1, 2, 1, 400, 150, gen.BSHD, True),      # Sq > Sk: first rows see no key
    (1, 2, 2, 100, 700, gen.BHSD, True),
    (1, 8, 2, 600, 1000, gen.BSHD, True),     # several query blocks, ragged tails
    (1, 4, 4, 300, 77, gen.BSHD, False),
]


@pytest.mark.parametrize("shape", SHAPES_D256, ids=lambda s: "d256_B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s"
                         % (s[0], s[1], s[2], s[3], s[4], "bshd" if s[5] == 0 else "bhsd",
                            "causal" if s[6] else "full"))
def test_prepped_equals_single_call_d256(shape):
    B, Hq, Hkv, Sq, Sk, layout, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=13 + Sq + Sk,
                           d=256)
    both(p)


SHAPES_D64 = [
    # head dim 64: 64-key tiles, 128 query rows per workgroup
    (1, 2, 2, 1, 1, gen.BSHD, False),
    (2, 4, 2, 63, 65, gen.BHSD, False),
    (1, 3, 3, 129, 127, gen.BSHD, True),
    (1, 2, 1, 400, 150, gen.BSHD, True),      # Sq > Sk: first rows see no key
    (1, 8, 2, 600, 1000, gen.BSHD, True),
    (1, 4, 4, 300, 77, gen.BHSD, False),
]


@pytest.mark.parametrize("shape", SHAPES_D64, ids=lambda s: "d64_B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s"
                         % (s[0], s[1], s[2], s[3], s[4], "bshd" if s[5] == 0 else "bhsd",
                            "causal" if s[6] else "full"))
def test_prepped_equals_single_call_d64(shape):
    B, Hq, Hkv, Sq, Sk, layout, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=17 + Sq + Sk,
                           d=64)
    both(p)


def test_prepped_d64_rounding_and_large_v():
    p = gen.prefill_inputs(1, 4, 2, 300, 500, layout=gen.BSHD, causal=True, seed=9, d=64)
    for rounding in ("rtna", "rtz"):
        both(p, rounding)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 40] = 3.0e5
    v[0, 333, 1, 9] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    both(p)


@pytest.mark.parametrize("rounding", ["rtne", "rtna", "rtz"])
def test_prepped_rounding_rules(rounding):
    p = gen.prefill_inputs(1, 4, 2, 300, 500, layout=gen.BSHD, causal=True, seed=5)
    both(p, rounding)


def test_prepped_v_beyond_fp16_range_takes_the_bf16_path():
    # infinities in the prepared tiles make the workgroup redo its rows with
    # bf16 V read from v itself, as the single-call forward does
    p = gen.prefill_inputs(1, 4, 2, 300, 1500, layout=gen.BSHD, causal=True, seed=83)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 5] = 3.0e5
    v[0, 700, 1, 9] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    both(p)


def test_prepped_d256_rounding_and_large_v():
    p = gen.prefill_inputs(1, 4, 2, 300, 500, layout=gen.BSHD, causal=True, seed=7, d=256)
    for rounding in ("rtna", "rtz"):
        both(p, rounding)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 200] = 3.0e5
    v[0, 333, 1, 9] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    both(p)


def test_prepared_tiles_serve_several_queries():
    # the tiles depend on v only: a second q runs on the same prepared tiles
    p = gen.prefill_inputs(2, 4, 4, 200, 600, layout=gen.BHSD, causal=False, seed=21)
    q, k, v, vt, kw = both(p)
    p2 = gen.prefill_inputs(2, 4, 4, 200, 600, layout=gen.BHSD, causal=False, seed=22)
    q2 = dev_bf16(p2.q)
    nvt = vt.numel()
    o_ref, l_ref = ea.attn_fwd(q2, k, v, prepare_v=False, **kw)
    o = torch.empty_like(q2)
    lse = torch.empty_like(l_ref)
    st = ea.library().attn_fwd_prepped(
        q2.data_ptr(), k.data_ptr(), v.data_ptr(), vt.data_ptr(), nvt, o.data_ptr(),
        lse.data_ptr(), p.B, p.Hq, p.Hkv, p.Sq, p.Sk, 128, float(p.scale), 0, ea.ATTN_BHSD, 0,
        None)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o_ref), bits_of(o))
    assert np.array_equal(l_ref.cpu().numpy().view(np.uint32), lse.cpu().numpy().view(np.uint32))


def test_prepared_gqa_tile_layout():
    # groups of 4k query heads: 32-key tiles, row d of 64 bytes holds keys
    # 32t + 16kk + {4hi..4hi+3, 8+4hi..8+4hi+3} at chunk (2kk + hi) ^ ((d >> 2) & 3)
    B, Hq, Hkv, Sk = 2, 8, 2, 50
    p = gen.prefill_inputs(B, Hq, Hkv, 1, Sk, layout=gen.BHSD, causal=False, seed=4)
    v = dev_bf16(p.v)
    nvt = ea.attn_prep_v_bytes(B, Hq, Hkv, Sk, 128)
    assert nvt == B * Hkv * 2 * 8192
    vt = torch.full((nvt,), 0x55, dtype=torch.uint8, device=v.device)
    st = ea.library().attn_prep_v(v.data_ptr(), B, Hq, Hkv, Sk, 128, ea.ATTN_BHSD, vt.data_ptr(),
                                  nvt, None)
    assert st == 0
    torch.cuda.synchronize()
    got = vt.cpu().numpy().view(np.float16).reshape(B, Hkv, 2, 128, 32)
    vf = (p.v.astype(np.uint32) << 16).view(np.float32)          # [B, Hkv, Sk, d]
    want = np.zeros((B, Hkv, 2, 128, 32), dtype=np.float16)
    for t in range(2):
        for d in range(128):
            for c in range(4):
                kk, hi = c >> 1, c & 1
                keys = [32 * t + 16 * kk + 4 * hi + j for j in range(4)] + \
                       [32 * t + 16 * kk + 8 + 4 * hi + j for j in range(4)]
                pc = c ^ ((d >> 2) & 3)
                for j, key in enumerate(keys):
                    if key < Sk:
                        want[:, :, t, d, 8 * pc + j] = vf[:, :, key, d].astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_prepared_tile_layout():
    # tile t of (b, h): row d holds keys 64t + 16kk + {4hi..4hi+3, 8+4hi..8+4hi+3}
    # at 16-byte chunk (2kk + hi) ^ ((d >> 1) & 7), as fp16; keys past Sk are 0
    B, Hq, Hkv, Sk = 2, 3, 3, 100
    p = gen.prefill_inputs(B, Hq, Hkv, 1, Sk, layout=gen.BSHD, causal=False, seed=3)
    v = dev_bf16(p.v)
    nvt = ea.attn_prep_v_bytes(B, Hq, Hkv, Sk, 128)
    vt = torch.full((nvt,), 0x55, dtype=torch.uint8, device=v.device)
    st = ea.library().attn_prep_v(v.data_ptr(), B, Hq, Hkv, Sk, 128, ea.ATTN_BSHD, vt.data_ptr(),
                                  nvt, None)
    assert st == 0
    torch.cuda.synchronize()
    got = vt.cpu().numpy().view(np.float16).reshape(B, Hkv, 2, 128, 64)
    vf = (p.v.astype(np.uint32) << 16).view(np.float32)          # [B, Sk, Hkv, d]
    want = np.zeros((B, Hkv, 2, 128, 64), dtype=np.float16)
    for t in range(2):
        for d in range(128):
            for c in range(8):
                kk, hi = c >> 1, c & 1
                keys = [64 * t + 16 * kk + 4 * hi + j for j in range(4)] + \
                       [64 * t + 16 * kk + 8 + 4 * hi + j for j in range(4)]
                pc = c ^ ((d >> 1) & 7)
                for j, key in enumerate(keys):
                    if key < Sk:
                        want[:, :, t, d, 8 * pc + j] = vf[:, key, :, d].astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_prepared_d256_tile_layout():
    # head dim 256: 32-key tiles of 16 KB, row d of 64 bytes holds keys
    # 32t + 16kk + {4hi..4hi+3, 8+4hi..8+4hi+3} at chunk (2kk + hi) ^ ((d >> 2) & 3)
    B, Hq, Hkv, Sk = 2, 2, 2, 40
    p = gen.prefill_inputs(B, Hq, Hkv, 1, Sk, layout=gen.BSHD, causal=False, seed=6, d=256)
    v = dev_bf16(p.v)
    nvt = ea.attn_prep_v_bytes(B, Hq, Hkv, Sk, 256)
    assert nvt == B * Hkv * 2 * 16384
    vt = torch.full((nvt,), 0x55, dtype=torch.uint8, device=v.device)
    st = ea.library().attn_prep_v(v.data_ptr(), B, Hq, Hkv, Sk, 256, ea.ATTN_BSHD, vt.data_ptr(),
                                  nvt, None)
    assert st == 0
    torch.cuda.synchronize()
    got = vt.cpu().numpy().view(np.float16).reshape(B, Hkv, 2, 256, 32)
    vf = (p.v.astype(np.uint32) << 16).view(np.float32)          # [B, Sk, Hkv, d]
    want = np.zeros((B, Hkv, 2, 256, 32), dtype=np.float16)
    for t in range(2):
        for d in range(256):
            for c in range(4):
                kk, hi = c >> 1, c & 1
                keys = [32 * t + 16 * kk + 4 * hi + j for j in range(4)] + \
                       [32 * t + 16 * kk + 8 + 4 * hi + j for j in range(4)]
                pc = c ^ ((d >> 2) & 3)
                for j, key in enumerate(keys):
                    if key < Sk:
                        want[:, :, t, d, 8 * pc + j] = vf[:, key, :, d].astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_prepared_d64_tile_layout():
    # head dim 64: tile t is the fp16 rows of keys 64t .. 64t+63 (128 bytes
    # each), 16-byte chunk c of row r at (c ^ s(r)) with
    # s(r) = ((r & 3) << 1) | ((r >> 2) & 1); keys past Sk are 0
    B, Hq, Hkv, Sk = 2, 2, 2, 100
    p = gen.prefill_inputs(B, Hq, Hkv, 1, Sk, layout=gen.BHSD, causal=False, seed=8, d=64)
    v = dev_bf16(p.v)
    nvt = ea.attn_prep_v_bytes(B, Hq, Hkv, Sk, 64)
    assert nvt == B * Hkv * 2 * 8192
    vt = torch.full((nvt,), 0x55, dtype=torch.uint8, device=v.device)
    st = ea.library().attn_prep_v(v.data_ptr(), B, Hq, Hkv, Sk, 64, ea.ATTN_BHSD, vt.data_ptr(),
                                  nvt, None)
    assert st == 0
    torch.cuda.synchronize()
    got = vt.cpu().numpy().view(np.float16).reshape(B, Hkv, 2, 64, 64)
    vf = (p.v.astype(np.uint32) << 16).view(np.float32)          # [B, Hkv, Sk, d]
    want = np.zeros((B, Hkv, 2, 64, 64), dtype=np.float16)
    for t in range(2):
        for r in range(64):
            key = 64 * t + r
            if key >= Sk:
                continue
            sw = ((r & 3) << 1) | ((r >> 2) & 1)
            for c in range(8):
                pc = c ^ sw
                want[:, :, t, r, 8 * pc:8 * pc + 8] = vf[:, :, key, 8 * c:8 * c + 8].astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
