"""The oracle at head dim 64: against torch's float64 attention (the
definition does not depend on d), the identical-keys closed form, and the
scale default 1/sqrt(d)."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import oracle.attention as att


@pytest.mark.parametrize("causal,layout,d", [(False, gen.BSHD, 64), (True, gen.BHSD, 64),
                                             (True, gen.BSHD, 256)])
def test_d64_matches_torch(causal, layout, d):
    p = gen.prefill_inputs(2, 4, 2, 40, 57, layout=layout, causal=causal, seed=41, d=d)
    assert p.q.shape[-1] == d and abs(p.scale - d ** -0.5) < 1e-12
    o, lse = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, causal, layout,
                           workers=1)
    f = [torch.from_numpy(np.ascontiguousarray(att._logical(att.bf16_to_f64(x), layout)))
         for x in (p.q, p.k, p.v)]
    q, k, v = f
    k, v = k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1)
    mask = None
    if causal:
        i = torch.arange(40)[:, None]
        j = torch.arange(57)[None, :]
        mask = j <= i + 17
    ot = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=p.scale)
    assert np.abs(o - ot.numpy()).max() <= 1e-12


def test_d64_identical_keys_give_the_mean_of_v():
    p = gen.prefill_inputs(1, 2, 1, 9, 33, layout=gen.BSHD, seed=42, d=64)
    k = np.ascontiguousarray(np.broadcast_to(p.k[:, :1], p.k.shape))
    o, lse = att.attention(p.q, k, p.v, 1, 2, 1, 9, 33, p.scale, False, gen.BSHD, workers=1)
    vmean = att.bf16_to_f64(p.v)[0, :, 0].mean(axis=0)
    assert np.abs(o[0] - vmean[None, None]).max() <= 1e-12
    s = p.scale * (att.bf16_to_f64(p.q)[0].transpose(1, 0, 2) @ att.bf16_to_f64(k)[0, 0, 0])
    assert np.abs(lse[0] - (s + np.log(33))).max() <= 1e-12
