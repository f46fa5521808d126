"""The decode entry point that allocates nothing (attn_decode_paged_noalloc,
for callers that cannot allocate device memory) gives, through the C ABI,
bitwise the result of the workspace entry point attn_decode_paged on the same
inputs, and meets the parity bound against the oracle, on consecutive calls of
decreasing then increasing size (the library's scratch array keeps the earlier
call's contents, which must not matter)."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from gpu_util import dev_bf16, dev_i32, host_f64, need_gpu
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(B, Hq, Hkv, L, seed):
    d = gen.decode_inputs(B, Hq, Hkv, max_len=L, seed=seed)
    return d, (dev_bf16(d.q), dev_bf16(d.k_pool), dev_bf16(d.v_pool), dev_i32(d.block_table),
               dev_i32(d.seq_lens))


def test_noalloc_equals_workspace_entry_on_consecutive_calls():
    # the decode workload's shape first, then a smaller problem, then a
    # mid-sized one: each reuses the array the previous call wrote
    for B, Hq, Hkv, L, seed in ((32, 32, 8, 4096, 5), (3, 8, 2, 300, 42), (9, 16, 4, 1500, 43)):
        print(f"case: noalloc B{B} Hq{Hq} Hkv{Hkv} L{L}", flush=True)
        d, (q, kp, vp, tab, lens) = _inputs(B, Hq, Hkv, L, seed)
        o1, l1 = ea.attn_decode_paged(q, kp, vp, tab, lens, scale=d.scale)
        o2 = torch.full_like(o1, float("nan"))
        l2 = torch.full_like(l1, float("nan"))
        st = ea.library().attn_decode_paged_noalloc(
            q.data_ptr(), kp.data_ptr(), vp.data_ptr(), tab.data_ptr(), lens.data_ptr(),
            o2.data_ptr(), l2.data_ptr(), B, Hq, Hkv, 128, 16, d.max_blocks, d.num_pages,
            float(d.scale), ctypes_stream())
        assert st == 0, ea.attn_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        o_ref, l_ref = att.decode_paged(d.q, d.k_pool, d.v_pool, d.block_table, d.seq_lens, d.Hkv,
                                        d.scale)
        e = check_o(host_f64(o2), o_ref, "noalloc decode")
        check_lse(host_f64(l2), l_ref, "noalloc decode lse")
        print(f"noalloc B{B}: bitwise equal to the workspace entry, err/tol {e[1]:.3f}",
              flush=True)


def test_binding_wrapper_and_size_limit():
    d, (q, kp, vp, tab, lens) = _inputs(4, 8, 2, 700, 44)
    o, l = ea.attn_decode_paged_noalloc(q, kp, vp, tab, lens, scale=d.scale)
    o1, l1 = ea.attn_decode_paged(q, kp, vp, tab, lens, scale=d.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(l, l1)
    # a problem whose partials exceed the array is refused before any launch
    big_tab = torch.zeros((64, 256), dtype=torch.int32, device=q.device)
    big_q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=q.device)
    big_lens = torch.ones(64, dtype=torch.int32, device=q.device)
    kc = torch.zeros((8, 16, 8, 128), dtype=torch.bfloat16, device=q.device)
    with pytest.raises(ValueError):
        ea.attn_decode_paged_noalloc(big_q, kc, kc, big_tab, big_lens)
    st = ea.library().attn_decode_paged_noalloc(
        big_q.data_ptr(), kc.data_ptr(), kc.data_ptr(), big_tab.data_ptr(), big_lens.data_ptr(),
        big_q.data_ptr(), l1.data_ptr(), 64, 32, 8, 128, 16, 256, 8, 0.1, ctypes_stream())
    assert st == -5


def ctypes_stream():
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
