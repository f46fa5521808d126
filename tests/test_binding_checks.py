"""The Python binding rejects caller-supplied outputs, workspaces and length
tensors that do not match what the kernels write or read, before anything
reaches the library (CPU only: tensors are stand-ins that carry a dtype, a
shape and a device, and the library is replaced by a stub that records
calls)."""
import math

import pytest
import torch

import exact_attention_60_amd as ea

BF, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
SIZE = {BF: 2, F32: 4, I32: 4, U8: 1}


class FakeT:
    """Just enough of a GPU tensor for the binding's checks."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contig = contiguous

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x10000

    def numel(self):
        return math.prod(self.shape)

    def element_size(self):
        return SIZE[self.dtype]


class Stream:
    cuda_stream = 0


class StubLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if name.startswith("attn_") and name.endswith("_bytes"):
            return lambda *a: 1 << 20
        def call(*a):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def lib(monkeypatch):
    stub = StubLib()
    monkeypatch.setattr(ea, "library", lambda: stub)
    return stub


B, S, H, HKV, D = 2, 64, 4, 2, 128


def fwd_args():
    q = FakeT((B, S, H, D), BF)
    k = FakeT((B, S, HKV, D), BF)
    return q, k, FakeT(k.shape, BF)


def good_fwd_out():
    return dict(out=FakeT((B, S, H, D), BF), lse=FakeT((B, H, S), F32))


BAD_OUT = [
    ("out", FakeT((B, S, H, D), F32)),                  # wrong dtype
    ("out", FakeT((B, S, H, D - 1), BF)),               # wrong shape
    ("out", FakeT((B, S - 1, H, D), BF)),               # undersized
    ("out", FakeT((B, S, H, D), BF, device="cpu")),     # host memory
    ("out", FakeT((B, S, H, D), BF, device="cuda:1")),  # another GPU
    ("out", FakeT((B, S, H, D), BF, contiguous=False)),
    ("lse", FakeT((B, H, S), BF)),
    ("lse", FakeT((B, S, H), F32)),
    ("lse", FakeT((B, H, S - 1), F32)),
    ("lse", FakeT((B, H, S), F32, contiguous=False)),
]


def good_vt():
    return FakeT((1 << 20,), U8)


def test_good_outputs_reach_the_library(lib):
    q, k, v = fwd_args()
    ea.attn_fwd(q, k, v, stream=Stream(), vt=good_vt(), prepare_v=True, **good_fwd_out())
    assert lib.calls == ["attn_prep_v", "attn_fwd_prepped"]
    lib.calls.clear()
    # default: 64 rows per head are one query tile, below the threshold
    ea.attn_fwd(q, k, v, stream=Stream(), **good_fwd_out())
    assert lib.calls == ["attn_fwd"]
    lib.calls.clear()
    ea.attn_fwd(q, k, v, stream=Stream(), prepare_v=False, **good_fwd_out())
    assert lib.calls == ["attn_fwd"]
    lib.calls.clear()
    ea.attn_fwd(q, k, v, stream=Stream(), prepare_v=False, rounding="rtz", **good_fwd_out())
    assert lib.calls == ["attn_fwd_rounded"]


@pytest.mark.parametrize("bad", [
    FakeT(((1 << 20) - 1,), U8),                 # too small
    FakeT((1 << 20,), U8, device="cpu"),         # host memory
    FakeT((1 << 20,), U8, device="cuda:1"),      # another GPU
    FakeT((1 << 20,), U8, contiguous=False),
])
def test_fwd_rejects_bad_vt(lib, bad):
    q, k, v = fwd_args()
    with pytest.raises(ValueError):
        ea.attn_fwd(q, k, v, stream=Stream(), vt=bad, prepare_v=True, **good_fwd_out())
    assert lib.calls == []


@pytest.mark.parametrize("name,bad", BAD_OUT)
def test_fwd_rejects_bad_outputs(lib, name, bad):
    q, k, v = fwd_args()
    kw = good_fwd_out()
    kw[name] = bad
    with pytest.raises(ValueError):
        ea.attn_fwd(q, k, v, stream=Stream(), **kw)
    with pytest.raises(ValueError):
        ea.attn_fwd(q, k, v, stream=Stream(), rounding="rtz", **kw)
    assert lib.calls == []


@pytest.mark.parametrize("name,bad", BAD_OUT)
def test_fp8_rejects_bad_outputs(lib, name, bad):
    q = FakeT((B, S, H, D), U8)
    k = FakeT((B, S, HKV, D), U8)
    kw = good_fwd_out()
    kw[name] = bad
    with pytest.raises(ValueError):
        ea.attn_fwd_fp8(q, k, FakeT(k.shape, U8), stream=Stream(), **kw)
    assert lib.calls == []


def test_inputs_on_another_device_are_rejected(lib):
    q, k, v = fwd_args()
    with pytest.raises(ValueError):
        ea.attn_fwd(q, FakeT(k.shape, BF, device="cuda:1"), v, stream=Stream(),
                    **good_fwd_out())
    assert lib.calls == []


def test_alibi_slopes_checked(lib):
    q, k, v = fwd_args()
    for bad in (FakeT((H + 1,), F32), FakeT((H,), BF), FakeT((H,), F32, device="cpu")):
        with pytest.raises(ValueError):
            ea.attn_fwd(q, k, v, stream=Stream(), alibi_slopes=bad, **good_fwd_out())
    assert lib.calls == []


def test_varlen_rejects_bad_outputs(lib):
    tq, tk = 100, 90
    q, k = FakeT((tq, H, D), BF), FakeT((tk, HKV, D), BF)
    cu = FakeT((B + 1,), I32)
    good = dict(out=FakeT((tq, H, D), BF), lse=FakeT((H, tq), F32))
    ea.attn_fwd_varlen(q, k, FakeT(k.shape, BF), cu, cu, 60, stream=Stream(), **good)
    assert lib.calls == ["attn_fwd_varlen"]
    for name, bad in (("out", FakeT((tq - 1, H, D), BF)), ("lse", FakeT((tq, H), F32)),
                      ("lse", FakeT((H, tq), BF))):
        kw = dict(good)
        kw[name] = bad
        with pytest.raises(ValueError):
            ea.attn_fwd_varlen(q, k, FakeT(k.shape, BF), cu, cu, 60, stream=Stream(), **kw)
    assert lib.calls == ["attn_fwd_varlen"]


def decode_args(seq_lens_n=B):
    q = FakeT((B, H, D), BF)
    kc = FakeT((10, 16, HKV, D), BF)
    return (q, kc, FakeT(kc.shape, BF), FakeT((B, 5), I32), FakeT((seq_lens_n,), I32))


def test_decode_good_outputs_reach_the_library(lib):
    ea.attn_decode_paged(*decode_args(), stream=Stream(), out=FakeT((B, H, D), BF),
                         lse=FakeT((B, H), F32), workspace=FakeT((1 << 20,), U8))
    assert lib.calls == ["attn_decode_paged"]


@pytest.mark.parametrize("kw", [
    dict(out=FakeT((B, H, D), F32)), dict(out=FakeT((B - 1, H, D), BF)),
    dict(lse=FakeT((B, H + 1), F32)), dict(lse=FakeT((B, H), BF)),
    dict(workspace=FakeT(((1 << 20) - 1,), U8)),           # too small
    dict(workspace=FakeT((1 << 20,), U8, device="cpu")),
    dict(workspace=FakeT((1 << 20,), U8, contiguous=False)),
])
def test_decode_rejects_bad_outputs(lib, kw):
    full = dict(out=FakeT((B, H, D), BF), lse=FakeT((B, H), F32),
                workspace=FakeT((1 << 20,), U8))
    full.update(kw)
    with pytest.raises(ValueError):
        ea.attn_decode_paged(*decode_args(), stream=Stream(), **full)
    assert lib.calls == []


@pytest.mark.parametrize("n", [B - 1, B + 1])
def test_decode_rejects_seq_lens_of_wrong_length(lib, n):
    with pytest.raises(ValueError):
        ea.attn_decode_paged(*decode_args(n), stream=Stream())
    assert lib.calls == []


def test_append_rows_checked(lib):
    for bad in (FakeT((B, HKV + 1, D), BF), FakeT((B, HKV, D), BF, device="cuda:1")):
        with pytest.raises(ValueError):
            ea.attn_decode_paged_append(decode_args()[0], bad, FakeT((B, HKV, D), BF),
                                        *decode_args()[1:], stream=Stream())
    assert lib.calls == []


def bwd_args():
    q, k, v = fwd_args()
    return q, k, v, FakeT(q.shape, BF), FakeT((B, H, S), F32), FakeT(q.shape, BF)


@pytest.mark.parametrize("name,bad", [
    ("dq", FakeT((B, S, H, D), F32)), ("dq", FakeT((B, S, HKV, D), BF)),
    ("dk", FakeT((B, S, H, D), BF)), ("dk", FakeT((B, S, HKV, D), BF, contiguous=False)),
    ("dv", FakeT((B, S, HKV, D - 64), BF)), ("dv", FakeT((B, S, HKV, D), BF, device="cpu")),
    ("workspace", FakeT((16,), U8)),
])
def test_bwd_rejects_bad_outputs(lib, name, bad):
    q, k, v, o, lse, do = bwd_args()
    kw = dict(dq=FakeT(q.shape, BF), dk=FakeT(k.shape, BF), dv=FakeT(v.shape, BF),
              workspace=FakeT((1 << 20,), U8))
    ea.attn_bwd(q, k, v, o, lse, do, stream=Stream(), **kw)
    assert lib.calls == ["attn_bwd"]
    kw[name] = bad
    with pytest.raises(ValueError):
        ea.attn_bwd(q, k, v, o, lse, do, stream=Stream(), **kw)
    assert lib.calls == ["attn_bwd"]


def test_bwd_varlen_rejects_bad_outputs(lib):
    tq, tk = 100, 90
    q, k = FakeT((tq, H, D), BF), FakeT((tk, HKV, D), BF)
    cu = FakeT((B + 1,), I32)
    args = (q, k, FakeT(k.shape, BF), FakeT(q.shape, BF), FakeT((H, tq), F32),
            FakeT(q.shape, BF), cu, cu, 60, 60)
    with pytest.raises(ValueError):
        ea.attn_bwd_varlen(*args, stream=Stream(), dq=FakeT(q.shape, BF),
                           dk=FakeT((tk + 1, HKV, D), BF), dv=FakeT(k.shape, BF))
    with pytest.raises(ValueError):
        ea.attn_bwd_varlen(*args, stream=Stream(), dq=FakeT((tq, H, D), F32),
                           dk=FakeT(k.shape, BF), dv=FakeT(k.shape, BF))
    assert lib.calls == []


def test_prepares_v_rule_per_head_dim():
    # d = 128: at least 32 query tiles of 256 rows per K/V head; d = 256: at
    # least 16 query blocks of 128 rows
    assert not ea.prepares_v(4, 32, 32, 4096, 4096, 128)      # 16 tiles
    assert ea.prepares_v(8, 32, 8, 8192, 8192, 128)           # 128 tiles
    assert ea.prepares_v(4, 32, 8, 4096, 4096, 256)           # 128 blocks
    assert ea.prepares_v(2, 16, 16, 4096, 4096, 256)          # 32 blocks
    assert ea.prepares_v(1, 4, 4, 2048, 2048, 256)            # 16 blocks
    assert not ea.prepares_v(4, 8, 8, 1024, 1024, 256)        # 8 blocks
    # d = 64: at least 32 query blocks of 128 rows
    assert ea.prepares_v(8, 32, 8, 8192, 8192, 64)            # 256 blocks
    assert ea.prepares_v(4, 32, 32, 4096, 4096, 64)           # 32 blocks
    assert not ea.prepares_v(4, 8, 8, 1024, 1024, 64)         # 8 blocks
