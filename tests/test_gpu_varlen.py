"""Parity of the packed-sequence forward (attn_fwd_varlen) and backward
(attn_bwd_varlen) with the fp64 oracles (GPU), under the forward's and the
backward's tolerances."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
import oracle.backward as obwd
from gpu_util import dev_bf16, dev_i32, host_f64, need_gpu
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(p, max_q=None, rounding="rtne"):
    o, lse = ea.attn_fwd_varlen(dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), dev_i32(p.cu_q),
                                dev_i32(p.cu_k), max_q or p.max_q, causal=p.causal,
                                scale=p.scale, rounding=rounding)
    torch.cuda.synchronize()
    return o, lse


def check(p, o, lse, what):
    o_ref, l_ref = att.attention_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, p.Hkv, p.scale, p.causal)
    e = check_o(host_f64(o), o_ref, what)
    el = check_lse(host_f64(lse), l_ref, what)
    print(f"{what}: max|dO| {e[0]:.3g} (err/tol {e[1]:.3f}) max|dLSE| {el:.3g}", flush=True)


@pytest.mark.parametrize("lq,lk,causal,Hq,Hkv", [
    ([5, 0, 17, 1, 33], [7, 3, 17, 1, 20], True, 4, 2),        # empty, tiny, Sq > Sk rows
    ([300, 256, 257, 1], [300, 256, 257, 1], True, 8, 2),     # tile edges, causal GQA
    ([12, 3, 0, 400], [30, 3, 8, 700], False, 4, 4),          # cross lengths, keys-only sequence
    ([513, 64], [0, 64], False, 2, 1),                        # a sequence with no keys at all
    ([1000, 37, 600], [1000, 37, 600], True, 4, 1),           # MQA, several query tiles
    # groups of 4k query heads: the GQA kernel (64-row tiles of four heads)
    ([5, 0, 17, 1, 65], [7, 3, 17, 1, 20], True, 8, 2),        # empty, tiny, Sq > Sk rows
    ([12, 3, 0, 400], [30, 3, 8, 700], False, 8, 2),          # cross lengths, keys-only sequence
    ([513, 64, 1], [0, 64, 1], False, 4, 1),                  # a sequence with no keys at all
    ([700, 129, 63], [700, 129, 63], True, 16, 2),            # groups of 8, ragged tails
])
def test_varlen_all_elements(lq, lk, causal, Hq, Hkv):
    p = gen.varlen_inputs(lq, lk, Hq, Hkv, causal=causal, seed=sum(lq) + sum(lk))
    o, lse = run(p)
    check(p, o, lse, f"varlen lq={lq} lk={lk} causal={causal}")


def test_varlen_max_seqlen_larger_than_needed_and_rounding():
    p = gen.varlen_inputs([100, 3], [90, 50], 4, 2, causal=True, seed=5)
    o1, l1 = run(p, max_q=2000)
    o2, l2 = run(p)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    check(p, o1, l1, "varlen max_seqlen 2000")
    o3, _ = run(p, rounding="rtz")
    check_o(host_f64(o3), att.attention_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, 2, p.scale,
                                               True)[0], "varlen rtz")


def test_varlen_equals_dense_per_sequence():
    """Each sequence of a packed batch gives bitwise the dense call's result on
    that sequence alone."""
    p = gen.varlen_inputs([200, 77, 300], [260, 77, 300], 4, 2, causal=True, seed=8)
    o, lse = run(p)
    for b in range(p.B):
        q0, q1, k0, k1 = (int(x) for x in (p.cu_q[b], p.cu_q[b + 1], p.cu_k[b], p.cu_k[b + 1]))
        od, ld = ea.attn_fwd(dev_bf16(p.q[q0:q1][None]), dev_bf16(p.k[k0:k1][None]),
                             dev_bf16(p.v[k0:k1][None]), causal=True, scale=p.scale, layout="bshd")
        torch.cuda.synchronize()
        assert torch.equal(od[0].view(torch.int16), o[q0:q1].view(torch.int16))
        assert torch.equal(ld[0], lse[:, q0:q1])


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2)], ids=["group2", "group4"])
def test_varlen_equals_dense_per_sequence_groups(Hq, Hkv):
    """Groups of 2 run the 8-wave kernel and groups of 4 the GQA kernel, in
    both calls: each sequence bitwise equals its dense call (V converted in
    the kernel, as the packed call does)."""
    p = gen.varlen_inputs([200, 77, 300, 1], [260, 77, 300, 40], Hq, Hkv, causal=True, seed=9)
    o, lse = run(p)
    for b in range(p.B):
        q0, q1, k0, k1 = (int(x) for x in (p.cu_q[b], p.cu_q[b + 1], p.cu_k[b], p.cu_k[b + 1]))
        od, ld = ea.attn_fwd(dev_bf16(p.q[q0:q1][None]), dev_bf16(p.k[k0:k1][None]),
                             dev_bf16(p.v[k0:k1][None]), causal=True, scale=p.scale, layout="bshd",
                             prepare_v=False)
        torch.cuda.synchronize()
        assert torch.equal(od[0].view(torch.int16), o[q0:q1].view(torch.int16)), b
        assert torch.equal(ld[0], lse[:, q0:q1]), b


def test_packed_prompt_batch_sampled():
    """The packed causal GQA batch of the benchmark (16 sequences up to 8192
    tokens): every row of a few (sequence, head) pairs."""
    p = gen.varlen_causal_gqa()
    o, lse = run(p)
    r = np.random.default_rng(0)
    for b in (int(np.argmax(np.diff(p.cu_q))), int(r.integers(p.B))):
        q0, q1 = int(p.cu_q[b]), int(p.cu_q[b + 1])
        k0, k1 = int(p.cu_k[b]), int(p.cu_k[b + 1])
        sub = gen.Varlen(p.q[q0:q1], p.k[k0:k1], p.v[k0:k1], np.array([0, q1 - q0], np.int32),
                         np.array([0, k1 - k0], np.int32), p.Hq, p.Hkv, True, p.scale)
        hs = [0, 31]
        o_ref, l_ref = att.attention_varlen(sub.q, sub.k, sub.v, sub.cu_q, sub.cu_k, p.Hkv,
                                            p.scale, True)
        check_o(host_f64(o[q0:q1, hs]), o_ref[:, hs], f"packed batch seq {b}")
        check_lse(host_f64(lse[hs, q0:q1]), l_ref[hs], f"packed batch seq {b} lse")


# ---- backward of packed sequences -------------------------------------------

def run_bwd(p, do_bits, max_q=None, max_k=None):
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    cq, ck = dev_i32(p.cu_q), dev_i32(p.cu_k)
    mq = max_q or p.max_q
    mk = max_k or max(1, int(np.diff(p.cu_k).max()))
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, ck, mq, causal=p.causal, scale=p.scale)
    g = ea.attn_bwd_varlen(q, k, v, o, lse, dev_bf16(do_bits), cq, ck, mq, mk, causal=p.causal,
                           scale=p.scale)
    torch.cuda.synchronize()
    return g


def packed_do(p, seed):
    r = np.random.default_rng(seed)
    return gen.f32_to_bf16_bits(r.standard_normal((int(p.cu_q[-1]), p.Hq, 128)).astype(np.float32))


@pytest.mark.parametrize("lq,lk,causal,Hq,Hkv", [
    ([5, 0, 17, 1, 33], [7, 3, 17, 1, 20], True, 4, 2),
    ([300, 256, 257, 1], [300, 256, 257, 1], True, 8, 2),
    ([12, 3, 0, 400], [30, 3, 8, 700], False, 4, 4),
    ([513, 64], [0, 64], False, 2, 1),
])
def test_varlen_backward_all_elements(lq, lk, causal, Hq, Hkv):
    from test_gpu_backward import check as check_grad
    p = gen.varlen_inputs(lq, lk, Hq, Hkv, causal=causal, seed=sum(lq) * 3 + 1)
    do = packed_do(p, 17)
    got = run_bwd(p, do)
    ref = obwd.attention_backward_varlen(p.q, p.k, p.v, do, p.cu_q, p.cu_k, Hkv, p.scale, causal,
                                         magnitudes=True)
    r = [check_grad(f"varlen {n}", host_f64(t), ref[i], ref[i + 3])
         for i, (n, t) in enumerate(zip(("dq", "dk", "dv"), got))]
    print(f"varlen backward lq={lq} lk={lk}: max err/tol {max(r):.3f}", flush=True)


def test_varlen_backward_equals_dense_per_sequence():
    p = gen.varlen_inputs([200, 77, 300], [260, 77, 300], 4, 2, causal=True, seed=9)
    do = packed_do(p, 9)
    dq, dk, dv = run_bwd(p, do)
    for b in range(p.B):
        q0, q1, k0, k1 = (int(x) for x in (p.cu_q[b], p.cu_q[b + 1], p.cu_k[b], p.cu_k[b + 1]))
        qs, ks, vs = (dev_bf16(x[None]) for x in (p.q[q0:q1], p.k[k0:k1], p.v[k0:k1]))
        od, ld = ea.attn_fwd(qs, ks, vs, causal=True, scale=p.scale, layout="bshd")
        g = ea.attn_bwd(qs, ks, vs, od, ld, dev_bf16(do[q0:q1][None]), causal=True,
                        scale=p.scale, layout="bshd")
        torch.cuda.synchronize()
        for x, y in zip(g, (dq[q0:q1], dk[k0:k1], dv[k0:k1])):
            assert torch.equal(x[0].view(torch.int16), y.view(torch.int16))
