"""Helpers for the GPU tests: move generator arrays to the device and back,
and compare against the oracle with the parity tolerance."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from tolerance import check_lse, check_o


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_fwd(p: gen.Prefill):
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    o, lse = ea.attn_fwd(q, k, v, causal=p.causal, scale=p.scale,
                         layout="bshd" if p.layout == gen.BSHD else "bhsd")
    torch.cuda.synchronize()
    return o, lse


def logical_o(o: torch.Tensor, layout: int) -> np.ndarray:
    """GPU output -> float64 [B, H, S, D]."""
    x = host_f64(o)
    return x.transpose(0, 2, 1, 3) if layout == gen.BSHD else x


def oracle_workers():
    """Host threads for the oracle beside a GPU test: one per core this
    process may use, at most 16 (one GPU's share of the host cores of an 8-GPU node)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def check_full(p: gen.Prefill, o, lse, what=""):
    o_ref, l_ref = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                 p.causal, p.layout, workers=oracle_workers())
    e_o = check_o(logical_o(o, p.layout), o_ref, what)
    e_l = check_lse(host_f64(lse), l_ref, what)
    return e_o, e_l


def sample_rows(p: gen.Prefill, n: int, seed: int):
    """Random (b, h, i) rows plus the edges of query tiles and of the tail."""
    r = np.random.default_rng(seed)
    rows = set()
    for _ in range(n):
        rows.add((int(r.integers(p.B)), int(r.integers(p.Hq)), int(r.integers(p.Sq))))
    for i in (0, 1, 63, 64, 255, 256, p.Sq - 1, p.Sq - 2, (p.Sq // 256) * 256 - 1):
        if 0 <= i < p.Sq:
            rows.add((p.B - 1, p.Hq - 1, i))
            rows.add((0, 0, i))
    for (b, s, h) in p.hot_rows:
        rows.add((b, h, s))
    return sorted(rows)


def check_sampled(p: gen.Prefill, o, lse, n=256, seed=0, what=""):
    rows = sample_rows(p, n, seed)
    o_ref, l_ref = att.attention_sampled(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                         p.causal, p.layout, rows, workers=oracle_workers())
    bsel = torch.tensor([r[0] for r in rows], device=o.device)
    hsel = torch.tensor([r[1] for r in rows], device=o.device)
    isel = torch.tensor([r[2] for r in rows], device=o.device)
    if p.layout == gen.BSHD:
        og = o[bsel, isel, hsel]
    else:
        og = o[bsel, hsel, isel]
    lg = lse[bsel, hsel, isel]
    e_o = check_o(host_f64(og), o_ref, what)
    e_l = check_lse(host_f64(lg), l_ref, what)
    return e_o, e_l
