"""The packed-sequence (variable-length) oracle against torch's float64
attention with a block-diagonal mask, against the dense oracle on one
sequence, and with planted mistakes that those pins must catch."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import attn_inputs as gen
import oracle.attention as att
import oracle.backward as obwd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def torch_packed(p):
    """float64 SDPA over the whole packed batch as one sequence with a mask
    that keeps each sequence to itself (bottom-right causal inside it)."""
    q = torch.from_numpy(att.bf16_to_f64(p.q)).permute(1, 0, 2)     # [Hq, Tq, D]
    k = torch.from_numpy(att.bf16_to_f64(p.k)).permute(1, 0, 2)
    v = torch.from_numpy(att.bf16_to_f64(p.v)).permute(1, 0, 2)
    G = p.Hq // p.Hkv
    k = k.repeat_interleave(G, dim=0)
    v = v.repeat_interleave(G, dim=0)
    Tq, Tk = int(p.cu_q[-1]), int(p.cu_k[-1])
    mask = torch.zeros((Tq, Tk), dtype=torch.bool)
    for b in range(p.B):
        q0, q1, k0, k1 = (int(x) for x in (p.cu_q[b], p.cu_q[b + 1], p.cu_k[b], p.cu_k[b + 1]))
        i = torch.arange(q1 - q0)[:, None]
        j = torch.arange(k1 - k0)[None, :]
        keep = (j <= i + (k1 - k0) - (q1 - q0)) if p.causal else torch.ones_like(i * j, dtype=bool)
        mask[q0:q1, k0:k1] = keep
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=float(np.float32(p.scale)))
    s = (q @ k.transpose(1, 2)) * float(np.float32(p.scale))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    seen = mask.any(dim=1).numpy()
    return o.permute(1, 0, 2).numpy(), lse.numpy(), seen


CASES = [
    ([5, 0, 17, 1, 33], [7, 3, 17, 1, 20], True, 4, 2),
    ([9, 16, 4], [9, 16, 4], True, 2, 1),
    ([12, 3, 0, 40], [30, 3, 8, 2], False, 4, 4),
]


@pytest.mark.parametrize("lq,lk,causal,Hq,Hkv", CASES)
def test_varlen_matches_torch_block_diagonal(lq, lk, causal, Hq, Hkv):
    p = gen.varlen_inputs(lq, lk, Hq, Hkv, causal=causal, seed=11)
    o, lse = att.attention_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, Hkv, p.scale, causal, workers=1)
    o_t, lse_t, seen = torch_packed(p)
    assert np.abs(o[seen] - o_t[seen]).max() <= 1e-12
    assert np.abs(lse[:, seen] - lse_t[:, seen]).max() <= 1e-12
    # rows that see no key (causal with more query rows than keys)
    assert np.all(o[~seen] == 0) and np.all(lse[:, ~seen] == -np.inf)


def test_one_sequence_equals_the_dense_oracle():
    p = gen.varlen_inputs([70], [90], 4, 2, causal=True, seed=3)
    o, lse = att.attention_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, 2, p.scale, True, workers=1)
    od, ld = att.attention(p.q[None], p.k[None], p.v[None], 1, 4, 2, 70, 90, p.scale, True,
                           att.BSHD, workers=1)
    assert np.array_equal(o, od[0].transpose(1, 0, 2)) and np.array_equal(lse, ld[0])


def test_empty_sequences_change_nothing():
    a = gen.varlen_inputs([6, 9], [6, 9], 2, 1, causal=True, seed=4)
    # the same two sequences with an empty one before each: the first empty
    # sequence owns 3 key rows (never attended), the second none
    pad = np.zeros((3, 1, 128), np.uint16)
    kb = np.concatenate([pad, a.k[:6], a.k[6:]])
    vb = np.concatenate([pad, a.v[:6], a.v[6:]])
    b = gen.Varlen(a.q, kb, vb, np.array([0, 0, 6, 6, 15], np.int32),
                   np.array([0, 3, 9, 9, 18], np.int32), 2, 1, True, a.scale)
    oa, la = att.attention_varlen(a.q, a.k, a.v, a.cu_q, a.cu_k, 1, a.scale, True, workers=1)
    ob, lb = att.attention_varlen(b.q, b.k, b.v, b.cu_q, b.cu_k, 1, b.scale, True, workers=1)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def fresh():
    spec = importlib.util.spec_from_file_location("varlen_mutant",
                                                  os.path.join(ROOT, "oracle", "attention.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _mut_global_causal(m):
    # causal alignment from packed positions instead of per sequence
    orig = m.attention_varlen

    def av(q, k, v, cu_q, cu_k, Hkv, scale, causal, workers=None):
        o, lse = orig(q, k, v, cu_q, cu_k, Hkv, scale, False, workers)
        if not causal:
            return o, lse
        Tq, Hq, d = q.shape
        for b in range(len(cu_q) - 1):
            q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
            nv = np.array([min(k1 - k0, max(0, q0 + i - k0 + 1)) for i in range(q1 - q0)])
            for h in range(Hq):
                g = m.kv_head_of(h, Hq, Hkv)
                oo, ll = m.attend_rows(m.bf16_to_f64(q[q0:q1, h]), m.bf16_to_f64(k[k0:k1, g]),
                                       m.bf16_to_f64(v[k0:k1, g]), m.scale_as_f32(scale), nv)
                o[q0:q1, h], lse[h, q0:q1] = oo, ll
        return o, lse
    m.attention_varlen = av


def _mut_keys_one_late(m):
    orig = m.attention_varlen
    m.attention_varlen = lambda q, k, v, cu_q, cu_k, *a, **kw: orig(
        q, k, v, cu_q, np.minimum(np.asarray(cu_k) + 1, len(k)), *a, **kw)


def _mut_shared_keys(m):
    # every sequence attends to the first sequence's keys
    orig = m.attention_varlen

    def av(q, k, v, cu_q, cu_k, *a, **kw):
        ck = np.asarray(cu_k).copy()
        return orig(q, np.concatenate([k[ck[0]:ck[1]]] * (len(ck) - 1)) if ck[1] > 0 else k,
                    np.concatenate([v[ck[0]:ck[1]]] * (len(ck) - 1)) if ck[1] > 0 else v,
                    cu_q, np.arange(len(ck)) * (ck[1] - ck[0]), *a, **kw)
    m.attention_varlen = av


@pytest.mark.parametrize("plant", [_mut_global_causal, _mut_keys_one_late, _mut_shared_keys],
                         ids=["global causal", "keys one late", "shared keys"])
def test_planted_varlen_mistake_is_caught(plant):
    m = fresh()
    plant(m)
    caught = False
    for lq, lk, causal, Hq, Hkv in CASES:
        p = gen.varlen_inputs(lq, lk, Hq, Hkv, causal=causal, seed=11)
        o, lse = m.attention_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, Hkv, p.scale, causal, workers=1)
        o_t, lse_t, seen = torch_packed(p)
        if not (np.abs(o[seen] - o_t[seen]).max() <= 1e-12 and
                np.abs(lse[:, seen] - lse_t[:, seen]).max() <= 1e-12):
            caught = True
    assert caught


def torch_packed_grads(p, do):
    """float64 autograd of sum(dO * O) through torch's attention over the
    packed batch with the block-diagonal mask (rows that see no key have
    zero output and are left out of the loss, as their O is 0)."""
    f = [torch.from_numpy(att.bf16_to_f64(x)).permute(1, 0, 2).contiguous()
         for x in (p.q, p.k, p.v, do)]
    q, k, v, dot = f
    for t in (q, k, v):
        t.requires_grad_(True)
    G = p.Hq // p.Hkv
    Tq, Tk = int(p.cu_q[-1]), int(p.cu_k[-1])
    mask = torch.zeros((Tq, Tk), dtype=torch.bool)
    for b in range(p.B):
        q0, q1, k0, k1 = (int(x) for x in (p.cu_q[b], p.cu_q[b + 1], p.cu_k[b], p.cu_k[b + 1]))
        i = torch.arange(q1 - q0)[:, None]
        j = torch.arange(k1 - k0)[None, :]
        mask[q0:q1, k0:k1] = (j <= i + (k1 - k0) - (q1 - q0)) if p.causal else True
    seen = mask.any(dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, dim=0), v.repeat_interleave(G, dim=0),
        attn_mask=mask | ~seen[:, None], scale=float(np.float32(p.scale)))
    (o[:, seen] * dot[:, seen]).sum().backward()
    return [t.grad.permute(1, 0, 2).numpy() for t in (q, k, v)]


@pytest.mark.parametrize("lq,lk,causal,Hq,Hkv", CASES)
def test_varlen_backward_matches_torch_autograd(lq, lk, causal, Hq, Hkv):
    p = gen.varlen_inputs(lq, lk, Hq, Hkv, causal=causal, seed=21)
    do = gen.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(
        (int(p.cu_q[-1]), Hq, 128)).astype(np.float32))
    got = obwd.attention_backward_varlen(p.q, p.k, p.v, do, p.cu_q, p.cu_k, Hkv, p.scale, causal,
                                         workers=1)
    ref = torch_packed_grads(p, do)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(g - r).max() / max(1e-300, np.abs(r).max())
        assert err <= 1e-12, f"{name}: relative error {err:.3g}"


def test_varlen_backward_one_sequence_equals_dense():
    p = gen.varlen_inputs([40], [57], 4, 2, causal=True, seed=22)
    do = gen.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((40, 4, 128)).astype(
        np.float32))
    a = obwd.attention_backward_varlen(p.q, p.k, p.v, do, p.cu_q, p.cu_k, 2, p.scale, True,
                                       workers=1)
    b = obwd.attention_backward(p.q[None], p.k[None], p.v[None], do[None], 1, 4, 2, 40, 57,
                                p.scale, True, att.BSHD, workers=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y[0].transpose(1, 0, 2))
