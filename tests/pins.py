"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each pin takes the oracle modules (``att`` = oracle.attention, ``onl`` =
oracle.online) as arguments so that the mutation tests can hand it a copy of
the oracle with a planted mistake and check that some pin catches it.

Facts used (none of them is the oracle's own formula retyped):
  P1  softmax rows sum to one                          (invariant)
  P2  identical keys give the mean of the visible V    (closed form)
  P3  one dominant logit selects its V row             (closed form)
  P4  causal row 0 is V[0]; causal row i is attention over the prefix;
      a single query row under the causal mask sees every key (decode)
  P5  the pages' blockwise online-softmax merge reproduces the oracle
  P6  split-KV partial merge is independent of the partition (incl. empty)
  P7  adding a vector u to every key shifts LSE by scale*q.u, O unchanged
  P8  permuting K and V rows together changes nothing (non-causal)
  P9  GQA equals MHA with each K/V head repeated for its query group
  P10 BSHD and BHSD copies of one problem agree
  P11 paged decode equals dense decode; page permutation changes nothing
  P12 torch CPU float64 scaled_dot_product_attention / logsumexp agree
  P13 a single key gives O = V[0], LSE = s_00
  P14 all-zero keys give O = mean(V), LSE = ln(Sk)
  P15 decode with a cache append equals torch float64 attention over the
      cached tokens before the current one followed by the new K/V row, and
      the pools change only in the current tokens' slots
"""
from __future__ import annotations

import math

import numpy as np

import attn_inputs as gen

D = 128
SC = 1.0 / math.sqrt(D)


def _bits(x):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return _bits(r.standard_normal(shape).astype(np.float32) * scale)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = (a == b) & np.isinf(a)
    bad = ~same_inf & ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    assert not bad.any(), f"{what}: max diff {np.nanmax(np.abs(a - b)[~same_inf])}"


# ----------------------------------------------------------------------------
def pin_p1_rows_sum_to_one(att, onl):
    r = np.random.default_rng(11)
    q = r.standard_normal((7, 16))
    k = r.standard_normal((23, 16)) * 3
    s = att.scores(q, k, 0.7)
    s[2, 5:] = -np.inf          # partly masked row
    p, m, l = att.row_softmax(s)
    tot = p.sum(axis=1)
    assert np.all(np.abs(tot - 1.0) <= 1e-12), tot
    assert np.all(p[2, 5:] == 0.0)
    assert np.all(p >= 0.0)
    # and the oracle's output is that P applied to V: a one-hot V column
    # extracts one column of P
    v = np.eye(23)[:, :16]
    o, _ = att.attend_rows(q, k, v, 0.7)
    full = np.zeros((7, 23))
    full[:] = att.row_softmax(att.scores(q, k, 0.7))[0]
    _close(o, full[:, :16], what="P1 columns")


def pin_p2_identical_keys(att, onl):
    """All keys of a KV head equal -> O_i = mean of visible V rows and
    LSE_i = scale*q_i.k + ln(#visible); distinct keys per KV head, so the GQA
    head mapping is exercised too."""
    B, Hq, Hkv, S = 2, 6, 3, 37
    r = np.random.default_rng(12)
    qf = _f64(_rand((B, S, Hq, D), 13))
    kv_vec = _f64(_rand((B, Hkv, D), 14))
    vf = _f64(_rand((B, S, Hkv, D), 15))
    kf = np.broadcast_to(kv_vec[:, None, :, :], (B, S, Hkv, D)).copy()
    for causal in (False, True):
        o, lse = att.attention(_bits(qf), _bits(kf), _bits(vf), B, Hq, Hkv, S, S,
                               SC, causal, gen.BSHD, chunk=8)
        sc = float(np.float32(SC))
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                for i in range(S):
                    n = i + 1 if causal else S
                    mean = vf[b, :n, g, :].mean(axis=0)
                    _close(o[b, h, i], mean, rtol=1e-12, atol=1e-13, what="P2 O")
                    s = sc * float(qf[b, i, h] @ kv_vec[b, g])
                    assert abs(lse[b, h, i] - (s + math.log(n))) <= 1e-11, "P2 LSE"
    del r


def pin_p3_dominant_logit(att, onl):
    r = np.random.default_rng(16)
    Sk = 50
    q = r.standard_normal(D)
    k = r.standard_normal((Sk, D)) * 0.01
    v = r.standard_normal((Sk, D))
    j = 31
    k[j] = q * (60.0 / (SC * (q @ q)))   # s_j = 60, the rest |s| < ~1
    o, lse = att.attend_rows(q[None], k, v, SC)
    s = SC * (k @ q)
    gap = s[j] - np.max(np.delete(s, j))
    assert gap >= 40
    bound = math.exp(-gap) * Sk * np.abs(v).max() * 2
    assert np.abs(o[0] - v[j]).max() <= bound, "P3 O"
    assert abs(lse[0] - s[j]) <= Sk * math.exp(-gap) * 2, "P3 LSE"


def pin_p4_causal(att, onl):
    B, H, S = 1, 3, 29
    q = _rand((B, H, S, D), 17)
    k = _rand((B, H, S, D), 18)
    v = _rand((B, H, S, D), 19)
    o, lse = att.attention(q, k, v, B, H, H, S, S, SC, True, gen.BHSD, chunk=5)
    sc = float(np.float32(SC))
    for h in range(H):
        assert np.array_equal(o[0, h, 0], _f64(v[0, h, 0])), "P4 row 0 must be V[0]"
        assert lse[0, h, 0] == sc * float(_f64(q[0, h, 0]) @ _f64(k[0, h, 0])), "P4 LSE0"
    for i in (1, 7, 28):
        op, lp = att.attention(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1],
                               B, H, H, 1, i + 1, SC, False, gen.BHSD)
        _close(o[:, :, i], op[:, :, 0], rtol=1e-12, atol=1e-14, what="P4 prefix O")
        _close(lse[:, :, i], lp[:, :, 0], what="P4 prefix LSE")
    # a single query row under the causal mask is decode: it sees every key
    o1, l1 = att.attention(q[:, :, 5:6], k, v, B, H, H, 1, S, SC, True, gen.BHSD)
    o2, l2 = att.attention(q[:, :, 5:6], k, v, B, H, H, 1, S, SC, False, gen.BHSD)
    _close(o1, o2, what="P4 Sq=1 causal")
    _close(l1, l2, what="P4 Sq=1 causal LSE")
    # more queries than keys: the first Sq-Sk rows see nothing
    o3, l3 = att.attention(q[:, :, :9], k[:, :, :4], v[:, :, :4], B, H, H, 9, 4, SC,
                           True, gen.BHSD)
    assert np.all(o3[:, :, :5] == 0) and np.all(l3[:, :, :5] == -np.inf), "P4 empty rows"
    assert np.array_equal(o3[:, :, 5], _f64(v[:, :, 0])), "P4 first visible row"


def pin_p5_online_blockwise(att, onl):
    r = np.random.default_rng(20)
    for Sk in (1, 5, 64, 130):
        k = r.standard_normal((Sk, D))
        v = r.standard_normal((Sk, D))
        q = r.standard_normal((4, D)) * np.array([1, 3, 8, 20])[:, None]
        o_ref, l_ref = att.attend_rows(q, k, v, SC)
        for blk in (1, 3, 16, 64, Sk):
            edges = list(range(0, Sk, blk)) + [Sk]
            for t in range(4):
                o, l = onl.online_attention_row(q[t], k, v, SC, edges)
                _close(o, o_ref[t], rtol=1e-12, atol=1e-13, what=f"P5 O blk={blk}")
                _close(l, l_ref[t], rtol=1e-12, atol=1e-12, what="P5 LSE")
        cuts = sorted(set(r.integers(0, Sk + 1, size=4).tolist()) | {0, Sk})
        o, l = onl.online_attention_row(q[2], k, v, SC, cuts)
        _close(o, o_ref[2], rtol=1e-12, atol=1e-13, what="P5 random cuts")


def pin_p6_split_merge(att, onl):
    r = np.random.default_rng(21)
    Sk = 77
    k = r.standard_normal((Sk, D))
    v = r.standard_normal((Sk, D))
    q = r.standard_normal((3, D)) * 4
    o_ref, l_ref = att.attend_rows(q, k, v, SC)
    for cuts in ([0, 77], [0, 10, 10, 77], [0, 1, 2, 40, 76, 77], [0, 0, 77, 77]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b > a:
                o, l = att.attend_rows(q, k[a:b], v[a:b], SC)
            else:
                o, l = np.zeros((3, D)), np.full(3, -np.inf)
            parts.append((o, l))
        for t in range(3):
            om, lm = onl.merge_partials([(p[0][t], p[1][t]) for p in parts])
            _close(om, o_ref[t], rtol=1e-12, atol=1e-13, what=f"P6 O {cuts}")
            _close(lm, l_ref[t], what="P6 LSE")


def pin_p7_key_shift(att, onl):
    r = np.random.default_rng(22)
    q = r.standard_normal((5, D))
    k = r.standard_normal((40, D))
    v = r.standard_normal((40, D))
    u = r.standard_normal(D) * 2
    o1, l1 = att.attend_rows(q, k, v, SC)
    o2, l2 = att.attend_rows(q, k + u, v, SC)
    _close(o2, o1, rtol=1e-10, atol=1e-12, what="P7 O")
    _close(l2, l1 + SC * (q @ u), rtol=1e-12, atol=1e-11, what="P7 LSE")


def pin_p8_permutation(att, onl):
    r = np.random.default_rng(23)
    q = r.standard_normal((6, D))
    k = r.standard_normal((33, D))
    v = r.standard_normal((33, D))
    perm = r.permutation(33)
    o1, l1 = att.attend_rows(q, k, v, SC)
    o2, l2 = att.attend_rows(q, k[perm], v[perm], SC)
    _close(o2, o1, rtol=1e-12, atol=1e-13, what="P8 O")
    _close(l2, l1, what="P8 LSE")


def pin_p9_gqa_is_repeated_mha(att, onl):
    B, Hq, S = 2, 8, 19
    for Hkv in (1, 2, 4):
        G = Hq // Hkv
        q = _rand((B, S, Hq, D), 24)
        k = _rand((B, S, Hkv, D), 25 + Hkv)
        v = _rand((B, S, Hkv, D), 35 + Hkv)
        o, l = att.attention(q, k, v, B, Hq, Hkv, S, S, SC, True, gen.BSHD)
        kr = np.repeat(k, G, axis=2)  # head h -> kv head h // G
        vr = np.repeat(v, G, axis=2)
        o2, l2 = att.attention(q, kr, vr, B, Hq, Hq, S, S, SC, True, gen.BSHD)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), f"P9 Hkv={Hkv}"
        # and the mapping is contiguous groups: head 0 and head G-1 share kv 0
        if G > 1:
            k2 = k.copy()
            k2[:, :, Hkv - 1] = 0  # change the last kv head only
            o3, _ = att.attention(q, k2, v, B, Hq, Hkv, S, S, SC, True, gen.BSHD)
            assert np.array_equal(o3[:, :Hq - G], o[:, :Hq - G]), "P9 groups"
            assert not np.array_equal(o3[:, Hq - G:], o[:, Hq - G:]), "P9 groups"


def pin_p10_layouts(att, onl):
    B, Hq, Hkv, Sq, Sk = 2, 4, 2, 23, 31
    q = _rand((B, Sq, Hq, D), 40)
    k = _rand((B, Sk, Hkv, D), 41)
    v = _rand((B, Sk, Hkv, D), 42)
    for causal in (False, True):
        o1, l1 = att.attention(q, k, v, B, Hq, Hkv, Sq, Sk, SC, causal, gen.BSHD)
        o2, l2 = att.attention(q.transpose(0, 2, 1, 3).copy(), k.transpose(0, 2, 1, 3).copy(),
                               v.transpose(0, 2, 1, 3).copy(), B, Hq, Hkv, Sq, Sk, SC,
                               causal, gen.BHSD)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "P10"
        # and head h of the BSHD problem is the (b, :, h, :) slice
        o3, l3 = att.attention(q[:, :, 1:2], k[:, :, 0:1], v[:, :, 0:1], B, 1, 1, Sq, Sk,
                               SC, causal, gen.BSHD)
        _close(o3[:, 0], o1[:, 1], what="P10 head slice")


def pin_p11_paged(att, onl):
    lens = [1, 16, 17, 40, 3]
    pa = gen.decode_inputs(5, 4, 2, max_len=48, seed=50, lens=lens, permute=True)
    pb = gen.decode_inputs(5, 4, 2, max_len=48, seed=50, lens=lens, permute=False)
    oa, la = att.decode_paged(pa.q, pa.k_pool, pa.v_pool, pa.block_table, pa.seq_lens, 2, SC)
    ob, lb = att.decode_paged(pb.q, pb.k_pool, pb.v_pool, pb.block_table, pb.seq_lens, 2, SC)
    # pools hold the same draws in page order; the permutation only moves pages
    # (the two pools differ, so compare against a dense re-layout of each)
    for p, o, l in ((pa, oa, la), (pb, ob, lb)):
        for b, n in enumerate(lens):
            # dense K/V: token t of seq b is page table[b, t//16], slot t%16
            pages = [p.block_table[b, t // 16] for t in range(n)]
            kd = np.stack([p.k_pool[pages[t], t % 16] for t in range(n)])  # [n, Hkv, D]
            vd = np.stack([p.v_pool[pages[t], t % 16] for t in range(n)])
            od, ld = att.attention(p.q[b][None, None], kd[None], vd[None], 1, 4, 2, 1, n, SC,
                                   False, gen.BSHD)
            _close(o[b], od[0, :, 0], what="P11 paged vs dense")
            _close(l[b], ld[0, :, 0], what="P11 LSE")
    # identity and permuted tables over the same logical data agree exactly
    perm = np.random.default_rng(51).permutation(pb.num_pages)
    inv = np.argsort(perm)
    kp = pb.k_pool[inv]
    vp = pb.v_pool[inv]       # page i of the new pool is old page inv[i]
    tab = pb.block_table.copy()
    valid = tab >= 0
    tab[valid] = perm[tab[valid]]
    oc, lc = att.decode_paged(pb.q, kp, vp, tab, pb.seq_lens, 2, SC)
    assert np.array_equal(oc, ob) and np.array_equal(lc, lb), "P11 permutation"
    assert np.all(np.isfinite(oa)) and np.all(np.isfinite(ob)), "P11 poison leaked"


def pin_p12_torch_sdpa(att, onl):
    import torch
    import torch.nn.functional as F
    r = np.random.default_rng(60)
    for Sq, Sk, causal in ((9, 9, True), (9, 9, False), (5, 13, False), (1, 7, False)):
        q = r.standard_normal((2, 3, Sq, D))
        k = r.standard_normal((2, 3, Sk, D))
        v = r.standard_normal((2, 3, Sk, D))
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.3).numpy()
        s = torch.matmul(qt, kt.transpose(-1, -2)) * 0.3
        if causal:
            s = s.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(1), float("-inf"))
        lt = torch.logsumexp(s, dim=-1).numpy()
        for b in range(2):
            for h in range(3):
                nv = [att.visible_keys(i, Sq, Sk, causal) for i in range(Sq)]
                o, l = att.attend_rows(q[b, h], k[b, h], v[b, h], 0.3, nv if causal else None)
                _close(o, ot[b, h], rtol=1e-10, atol=1e-12, what="P12 O")
                _close(l, lt[b, h], rtol=1e-12, atol=1e-12, what="P12 LSE")


def pin_p15_append(att, onl):
    import torch
    import torch.nn.functional as F
    lens = [1, 16, 17, 33, 2]
    p = gen.decode_append_inputs(5, 6, 2, max_len=48, seed=90, lens=lens)
    d = p.base
    o, l, kp, vp = att.decode_paged_append(d.q, p.k_new, p.v_new, d.k_pool, d.v_pool,
                                           d.block_table, d.seq_lens, 2, SC)
    sc = float(np.float32(SC))
    for b, n in enumerate(lens):
        # the tokens cached before the current one, read through the table of
        # the pools as they were, then the current token's rows
        old_k = [d.k_pool[d.block_table[b, t // 16], t % 16] for t in range(n - 1)]
        old_v = [d.v_pool[d.block_table[b, t // 16], t % 16] for t in range(n - 1)]
        kd = _f64(np.stack(old_k + [p.k_new[b]]))          # [n, Hkv, D]
        vd = _f64(np.stack(old_v + [p.v_new[b]]))
        for h in range(6):
            g = h // 3
            qt = torch.from_numpy(_f64(d.q[b, h]))[None, None, None]
            kt = torch.from_numpy(kd[:, g])[None, None]
            vt = torch.from_numpy(vd[:, g])[None, None]
            ot = F.scaled_dot_product_attention(qt, kt, vt, scale=sc)[0, 0, 0].numpy()
            lt = torch.logsumexp(torch.matmul(qt, kt.transpose(-1, -2)) * sc, dim=-1).item()
            _close(o[b, h], ot, rtol=1e-10, atol=1e-12, what="P15 O")
            _close(l[b, h], lt, rtol=1e-12, atol=1e-12, what="P15 LSE")
    # the pools: only the current tokens' slots change, to the new rows
    for pool, new, upd in ((d.k_pool, p.k_new, kp), (d.v_pool, p.v_new, vp)):
        changed = np.zeros(pool.shape[:2], bool)
        for b, n in enumerate(lens):
            pg, sl = d.block_table[b, (n - 1) // 16], (n - 1) % 16
            changed[pg, sl] = True
            assert np.array_equal(upd[pg, sl], new[b]), "P15 new row"
        assert np.array_equal(upd[~changed], pool[~changed]), "P15 other slots"
    assert np.all(np.isfinite(o)), "P15 the stale slot leaked"


def pin_p13_single_key(att, onl):
    q = _rand((1, 3, 1, D), 70)
    k = _rand((1, 3, 1, D), 71)
    v = _rand((1, 3, 1, D), 72)
    q5 = np.repeat(q, 5, axis=2)
    o, l = att.attention(q5, k, v, 1, 3, 3, 5, 1, SC, False, gen.BHSD)
    sc = float(np.float32(SC))
    for h in range(3):
        for i in range(5):
            assert np.array_equal(o[0, h, i], _f64(v[0, h, 0])), "P13 O"
            assert l[0, h, i] == sc * float(_f64(q[0, h, 0]) @ _f64(k[0, h, 0])), "P13 LSE"


def pin_p14_zero_keys(att, onl):
    B, H, Sq, Sk = 1, 2, 6, 24
    q = _rand((B, H, Sq, D), 80, 5.0)
    k = np.zeros((B, H, Sk, D), np.uint16)
    v = _rand((B, H, Sk, D), 81)
    o, l = att.attention(q, k, v, B, H, H, Sq, Sk, SC, False, gen.BHSD)
    mean = _f64(v).mean(axis=2)
    for i in range(Sq):
        _close(o[:, :, i], mean, rtol=1e-12, atol=1e-13, what="P14 O")
        _close(l[:, :, i], np.full((B, H), math.log(Sk)), what="P14 LSE")


ALL_PINS = [pin_p1_rows_sum_to_one, pin_p2_identical_keys, pin_p3_dominant_logit,
            pin_p4_causal, pin_p5_online_blockwise, pin_p6_split_merge,
            pin_p7_key_shift, pin_p8_permutation, pin_p9_gqa_is_repeated_mha,
            pin_p10_layouts, pin_p11_paged, pin_p12_torch_sdpa, pin_p15_append,
            pin_p13_single_key,
            pin_p14_zero_keys]
