"""Pins of the backward oracle: each takes an oracle module (the real one or a
copy with a planted mistake) and raises AssertionError when it disagrees with
what the mathematics fixes.  Used by test_oracle_backward.py and by the
mutation tests."""
import numpy as np
import torch

import attn_inputs as gen
import oracle.attention as att

BSHD, BHSD = gen.BSHD, gen.BHSD


def _logical(x, layout):
    return x.transpose(0, 2, 1, 3) if layout == BSHD else x


def _loss(q, k, v, do, B, Hq, Hkv, Sq, Sk, scale, causal, layout, slopes=None):
    """L = sum(dO * O) with O from the forward oracle's attend_rows (float64
    inputs), with the ALiBi bias of the given slopes."""
    ql, kl, vl, dol = (_logical(x, layout) for x in (q, k, v, do))
    nv = np.array([att.visible_keys(i, Sq, Sk, causal) for i in range(Sq)])
    total = 0.0
    for b in range(B):
        for h in range(Hq):
            g = att.kv_head_of(h, Hq, Hkv)
            bias = None if slopes is None else att.alibi_bias(np.arange(Sq), Sq, Sk, slopes[h])
            o, _ = att.attend_rows(ql[b, h], kl[b, g], vl[b, g], float(np.float32(scale)), nv,
                                   bias)
            total += float((o * dol[b, h]).sum())
    return total


def finite_difference(bwd, B=1, Hq=4, Hkv=2, Sq=5, Sk=7, d=8, causal=False, layout=BSHD,
                      seed=0, eps=1e-6, tol=1e-7, slopes=None):
    """Central differences of L = sum(dO * O) (forward oracle, float64) against
    the analytic gradient, every entry of dQ, dK and dV (with ALiBi when
    slopes are given)."""
    r = np.random.default_rng(seed)
    q = r.standard_normal(gen.layout_shape(layout, B, Hq, Sq, d))
    k = r.standard_normal(gen.layout_shape(layout, B, Hkv, Sk, d))
    v = r.standard_normal(gen.layout_shape(layout, B, Hkv, Sk, d))
    do = r.standard_normal(gen.layout_shape(layout, B, Hq, Sq, d))
    scale = 0.375  # exact in float32
    args = (B, Hq, Hkv, Sq, Sk, scale, causal, layout)
    dq, dk, dv = bwd.attention_backward(q, k, v, do, *args, workers=1, alibi_slopes=slopes)
    for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, *args, slopes)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, *args, slopes)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(_logical(num, layout) - g).max()
        assert err <= tol, f"finite differences: {name} off by {err:.3g}"


def torch_autograd(bwd, B=2, Hq=4, Hkv=2, Sq=33, Sk=70, causal=True, layout=BHSD, seed=7):
    """torch float64 autograd through its scaled_dot_product_attention with an
    explicit bottom-right causal mask and K/V heads repeated per group."""
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=seed)
    do = gen.output_grad(p, seed)
    dq, dk, dv = bwd.attention_backward(p.q, p.k, p.v, do, B, Hq, Hkv, Sq, Sk, p.scale, causal,
                                        layout, workers=1)
    t = [torch.from_numpy(np.ascontiguousarray(_logical(att.bf16_to_f64(x), layout)))
         for x in (p.q, p.k, p.v, do)]
    qt, kt, vt, dot = t
    qt.requires_grad_(True), kt.requires_grad_(True), vt.requires_grad_(True)
    G = Hq // Hkv
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    mask = None
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        mask = j <= i + (Sk - Sq)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kr, vr, attn_mask=mask, scale=float(np.float32(p.scale)))
    (o * dot).sum().backward()
    for name, ref, got in (("dq", qt.grad, dq), ("dk", kt.grad, dk), ("dv", vt.grad, dv)):
        ref = ref.numpy()
        err = np.abs(ref - got).max() / max(1e-300, np.abs(ref).max())
        assert err <= 1e-12, f"torch autograd: {name} relative error {err:.3g}"


def _problem(B=2, Hq=4, Hkv=2, Sq=40, Sk=57, causal=False, layout=BSHD, seed=3, **kw):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=seed, **kw)
    return p, gen.output_grad(p, seed)


def invariants(bwd, causal=False, layout=BSHD, Sq=40, Sk=57):
    """Identities of the exact gradient, per (batch, K/V head g), summing over
    the query heads of g:
      shift invariance of the keys   sum_j dK_j = 0
      rows of P sum to one           sum_j dV_j = sum of dO over rows that see a key
      O is linear in V               sum <dV_j, V_j> = sum <dO_i, O_i>
      S depends on Q K^T only        sum <dQ_i, Q_i> = sum <dK_j, K_j>"""
    p, do = _problem(Sq=Sq, Sk=Sk, causal=causal, layout=layout)
    dq, dk, dv = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                        p.causal, p.layout, workers=1)
    o, _ = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal,
                         p.layout, workers=1)
    q, k, v, dof = (_logical(att.bf16_to_f64(x), p.layout) for x in (p.q, p.k, p.v, do))
    G = p.Hq // p.Hkv
    seen = np.array([att.visible_keys(i, p.Sq, p.Sk, p.causal) > 0 for i in range(p.Sq)])
    for b in range(p.B):
        for g in range(p.Hkv):
            hs = slice(g * G, (g + 1) * G)
            sdk = dk[b, g].sum(axis=0)
            assert np.abs(sdk).max() <= 1e-12 * max(1.0, np.abs(dk[b, g]).sum()), \
                "sum of dK over keys must vanish"
            sdv = dv[b, g].sum(axis=0)
            sdo = dof[b, hs][:, seen].sum(axis=(0, 1))
            assert np.allclose(sdv, sdo, rtol=0, atol=1e-11), "sum of dV must equal sum of dO"
            lhs = (dv[b, g] * v[b, g]).sum()
            rhs = (dof[b, hs] * o[b, hs]).sum()
            assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs)), "<dV,V> must equal <dO,O>"
            lq = (dq[b, hs] * q[b, hs]).sum()
            lk = (dk[b, g] * k[b, g]).sum()
            assert abs(lq - lk) <= 1e-10 * max(1.0, abs(lk)), "<dQ,Q> must equal <dK,K>"


def special_cases(bwd):
    """Closed forms: one key (O = V_0 for every row: dQ = dK = 0 and
    dV_0 = sum of dO); identical keys (P uniform for every Q: dQ = 0); rows
    that see no key (causal Sq > Sk: dQ = 0 there, and the result equals the
    problem restricted to the other rows)."""
    p, do = _problem(Sq=9, Sk=1, layout=BHSD)
    dq, dk, dv = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                        False, p.layout, workers=1)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13, "Sk=1: dQ, dK must be 0"
    dof = att.bf16_to_f64(do)
    G = p.Hq // p.Hkv
    for g in range(p.Hkv):
        ref = dof[:, g * G:(g + 1) * G].sum(axis=(1, 2))
        assert np.abs(dv[:, g, 0] - ref).max() <= 1e-12, "Sk=1: dV_0 must be the sum of dO"

    p = gen.equal_keys_prefill(2, 4, 2, 24, 50, layout=BSHD, seed=5)
    do = gen.output_grad(p, 5)
    dq, _, _ = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                      False, p.layout, workers=1)
    assert np.abs(dq).max() <= 1e-12, "identical keys: dQ must be 0"

    Sq, Sk = 30, 12
    p, do = _problem(Sq=Sq, Sk=Sk, causal=True, layout=BHSD)
    dq, dk, dv = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, Sq, Sk, p.scale,
                                        True, p.layout, workers=1)
    empty = Sq - Sk
    assert np.all(dq[:, :, :empty] == 0), "rows with no visible key: dQ must be 0"
    q2, do2 = p.q[:, :, empty:], do[:, :, empty:]
    dq2, dk2, dv2 = bwd.attention_backward(q2, p.k, p.v, do2, p.B, p.Hq, p.Hkv, Sk, Sk, p.scale,
                                           True, p.layout, workers=1)
    assert np.abs(dq2 - dq[:, :, empty:]).max() <= 1e-13
    assert np.abs(dk2 - dk).max() <= 1e-13 and np.abs(dv2 - dv).max() <= 1e-13, \
        "empty rows must add nothing to dK, dV"


def layouts_and_groups(bwd):
    """BSHD and BHSD copies of one problem give the same gradients, and GQA
    equals MHA on K/V heads repeated per group with dK, dV summed back."""
    pb, dob = _problem(Sq=21, Sk=35, causal=True, layout=BSHD, Hq=6, Hkv=2)
    a = bwd.attention_backward(pb.q, pb.k, pb.v, dob, pb.B, 6, 2, 21, 35, pb.scale, True, BSHD,
                               workers=1)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))  # noqa: E731
    b = bwd.attention_backward(t(pb.q), t(pb.k), t(pb.v), t(dob), pb.B, 6, 2, 21, 35, pb.scale,
                               True, BHSD, workers=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "BSHD and BHSD must agree"
    rep = lambda x: np.ascontiguousarray(np.repeat(x, 3, axis=2))  # noqa: E731
    m = bwd.attention_backward(pb.q, rep(pb.k), rep(pb.v), dob, pb.B, 6, 6, 21, 35, pb.scale,
                               True, BSHD, workers=1)
    assert np.abs(m[0] - a[0]).max() <= 1e-13, "GQA dQ must equal MHA's"
    for gm, ga in ((m[1], a[1]), (m[2], a[2])):
        summed = gm.reshape(pb.B, 2, 3, 35, -1).sum(axis=2)
        assert np.abs(summed - ga).max() <= 1e-12, "GQA dK/dV must be MHA's summed per group"


ALL = [
    ("finite differences, non-causal BSHD", lambda m: finite_difference(m)),
    ("finite differences, causal BHSD", lambda m: finite_difference(m, causal=True, layout=BHSD)),
    ("finite differences, causal Sq > Sk", lambda m: finite_difference(m, Sq=7, Sk=4, causal=True)),
    ("finite differences, ALiBi causal", lambda m: finite_difference(
        m, Sq=6, Sk=9, causal=True, slopes=np.array([0.5, 0.25, 0.125, 0.0625], np.float32))),
    ("finite differences, ALiBi cross", lambda m: finite_difference(
        m, Sq=7, Sk=4, layout=BHSD, slopes=np.array([1.0, 0.5, 0.3, 0.2], np.float32))),
    ("torch autograd", lambda m: torch_autograd(m)),
    ("invariants", lambda m: invariants(m)),
    ("invariants causal", lambda m: invariants(m, causal=True, layout=BHSD)),
    ("special cases", special_cases),
    ("layouts and groups", layouts_and_groups),
]
