"""The C-ABI library loads, exports what include/attn.h declares, and rejects
invalid arguments before any HIP call (CPU only: no kernel is launched)."""
import ctypes
import os
import re

import pytest

import exact_attention_60_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ea.library()
    declared = header_functions()
    assert set(declared) == set(ea.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    # and they are real dynamic symbols of the .so
    out = os.popen(f"nm -D --defined-only {ea.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings():
    assert ea.attn_version() == 13
    for code in ea.STATUS:
        assert ea.attn_status_string(code)
    assert ea.attn_status_string(12345) == "unknown status"


def test_workspace_bytes():
    # B * Hq * (S * (128 + 1) + 1) floats with S = ceil(max_blocks / 4) + 1
    # partial results per (sequence, head), plus one count per (sequence, head)
    assert ea.attn_decode_workspace_bytes(32, 32, 256) == 32 * 32 * (65 * 129 + 1) * 4
    assert ea.attn_decode_workspace_bytes(2, 3, 9) == 2 * 3 * (4 * 129 + 1) * 4
    assert ea.attn_decode_workspace_bytes(1, 1, 1) == (2 * 129 + 1) * 4
    assert ea.attn_decode_workspace_bytes(0, 1, 1) == 0
    assert ea.attn_decode_workspace_bytes(1, 1, 0) == 0


P = 0x10000  # a fake, 16-byte aligned "device" pointer: never dereferenced


def fwd(rounding=None, **kw):
    """attn_fwd, or attn_fwd_rounded when a rounding code is given."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1,
             causal=0, layout=0, stream=None)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
            a["d"], a["scale"], a["causal"], a["layout"])
    if rounding is None:
        return ea.library().attn_fwd(*args, a["stream"])
    return ea.library().attn_fwd_rounded(*args, rounding, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(v=None), -1),
    (dict(B=0), -2), (dict(Sq=0), -2), (dict(Sk=-1), -2), (dict(Hq=3, Hkv=2), -2),
    (dict(d=96), -3), (dict(d=512), -3), (dict(layout=2), -3), (dict(causal=2), -3),
    (dict(scale=0.0), -3), (dict(scale=float("nan")), -3), (dict(scale=float("inf")), -3),
    (dict(scale=-1.0), -3),
    (dict(q=P + 8), -4), (dict(o=P + 2), -4), (dict(lse=P + 4), -4),
    (dict(Sk=(1 << 22) + 1, Hkv=2, Hq=2, layout=0), -2),   # K/V of one head exceed 32-bit offsets
])
def test_fwd_argument_errors(kw, code):
    assert fwd(**kw) == code
    for r in (0, 1, 2):                      # the rounded variant checks the same
        assert fwd(rounding=r, **kw) == code


def test_prep_v_bytes():
    tile = 64 * 128 * 2
    # B * Hkv * ceil(Sk / 64) tiles of 16 KB where the prefill kernel reads them
    assert ea.attn_prep_v_bytes(2, 4, 2, 100, 128) == 2 * 2 * 2 * tile
    assert ea.attn_prep_v_bytes(4, 32, 32, 4096, 128) == 4 * 32 * 64 * tile
    assert ea.attn_prep_v_bytes(1, 6, 3, 64, 128) == 3 * 1 * tile
    assert ea.attn_prep_v_bytes(1, 1, 1, 65, 128) == 2 * tile
    # groups of 4k query heads: the GQA kernel's tiles of 32 keys (8 KB)
    assert ea.attn_prep_v_bytes(2, 8, 2, 100, 128) == 2 * 2 * 4 * 8192
    assert ea.attn_prep_v_bytes(8, 32, 8, 8192, 128) == 8 * 8 * 256 * 8192
    assert ea.attn_prep_v_bytes(1, 4, 1, 32, 128) == 8192
    # head dim 256: tiles of 32 keys (16 KB) for every group size
    assert ea.attn_prep_v_bytes(2, 4, 4, 100, 256) == 2 * 4 * 4 * 16384
    assert ea.attn_prep_v_bytes(4, 32, 8, 4096, 256) == 4 * 8 * 128 * 16384
    assert ea.attn_prep_v_bytes(1, 3, 1, 32, 256) == 16384
    # head dim 64: tiles of 64 keys (8 KB)
    assert ea.attn_prep_v_bytes(2, 4, 4, 100, 64) == 2 * 4 * 2 * 8192
    assert ea.attn_prep_v_bytes(8, 32, 8, 8192, 64) == 8 * 8 * 128 * 8192
    # none for other head dims
    assert ea.attn_prep_v_bytes(2, 4, 4, 100, 96) == 0
    # invalid sizes
    assert ea.attn_prep_v_bytes(0, 4, 4, 100, 128) == 0
    assert ea.attn_prep_v_bytes(1, 3, 2, 100, 128) == 0
    assert ea.attn_prep_v_bytes(1, 4, 4, 0, 128) == 0


def prep(**kw):
    a = dict(v=P, B=1, Hq=4, Hkv=2, Sk=8, d=128, layout=0, vt=P, vtb=1 << 40, stream=None)
    a.update(kw)
    return ea.library().attn_prep_v(a["v"], a["B"], a["Hq"], a["Hkv"], a["Sk"], a["d"],
                                    a["layout"], a["vt"], a["vtb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), -1), (dict(B=0), -2), (dict(Hq=3, Hkv=2), -2), (dict(Sk=0), -2),
    (dict(layout=2), -3), (dict(vt=None), -5), (dict(vtb=16384 * 2 - 1), -5),
    (dict(v=P + 2), -4), (dict(vt=P + 8), -4),
    (dict(Sk=(1 << 24) + 1), -2),                  # one head's tiles exceed 32-bit offsets
    (dict(d=256, Sk=(1 << 23) + 1), -2),
    (dict(d=64, vt=None), -5), (dict(d=64, vtb=2 * 8192 - 1), -5),
    (dict(d=256, vt=None), -5), (dict(d=256, vtb=2 * 16384 - 1), -5), (dict(d=256, vt=P + 8), -4),
])
def test_prep_v_argument_errors(kw, code):
    assert prep(**kw) == code


def test_prep_v_without_tiles_is_a_no_op():
    # shapes that do not use the tiles return at once (no device call)
    assert prep(d=96, vt=None, vtb=0) == 0
    # groups of 4k heads use them (32-key tiles)
    assert prep(Hq=8, Hkv=2, vt=None, vtb=0) == -5
    assert prep(Hq=8, Hkv=2, vtb=8192 - 1) == -5


def prepped(rounding=0, vt=P, vtb=1 << 62, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1,
             causal=0, layout=0, stream=None)
    a.update(kw)
    return ea.library().attn_fwd_prepped(
        a["q"], a["k"], a["v"], vt, vtb, a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
        a["Sk"], a["d"], a["scale"], a["causal"], a["layout"], rounding, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(vt=None), -1), (dict(vtb=16384 * 2 - 1), -5), (dict(vt=P + 8), -4),
    (dict(Sk=(1 << 24) + 1, Hkv=4), -2),
    # the tiles are ignored where the shape does not use them
    (dict(vt=None, d=96), -3),
    (dict(vt=None, d=64), -1), (dict(d=64, vtb=2 * 8192 - 1), -5),
    (dict(vt=None, Hq=8, Hkv=2), -1), (dict(Hq=8, Hkv=2, vtb=8191), -5),
    (dict(vt=None, d=256), -1), (dict(d=256, vtb=2 * 16384 - 1), -5),
    (dict(d=256, Sk=(1 << 23) + 1, Hkv=4), -2),
])
def test_fwd_prepped_argument_errors(kw, code):
    assert prepped(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(B=0), -2), (dict(Hq=3, Hkv=2), -2),
    (dict(d=96), -3), (dict(layout=2), -3), (dict(scale=float("nan")), -3), (dict(o=P + 2), -4),
    (dict(Sk=(1 << 22) + 1, Hkv=2, Hq=2, layout=0), -2),
])
def test_fwd_prepped_checks_like_fwd(kw, code):
    assert fwd(**kw) == code
    for r in (0, 1, 2):
        assert prepped(rounding=r, **kw) == code
    assert prepped(rounding=3) == -3


@pytest.mark.parametrize("r", [-1, 3, 100])
def test_unknown_rounding_rule_is_unsupported(r):
    assert fwd(rounding=r) == -3
    assert dec(rounding=r) == -3


def dec(rounding=None, **kw):
    """attn_decode_paged, or attn_decode_paged_rounded when a rounding code is
    given."""
    a = dict(q=P, k=P, v=P, tab=P, lens=P, o=P, lse=P, B=2, Hq=8, Hkv=2, d=128, page=16,
             mb=4, npages=8, scale=0.1, ws=P, wsb=10 ** 6, stream=None)
    a.update(kw)
    head = (a["q"], a["k"], a["v"], a["tab"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"],
            a["Hkv"], a["d"], a["page"], a["mb"], a["npages"], a["scale"])
    tail = (a["ws"], a["wsb"], a["stream"])
    if rounding is None:
        return ea.library().attn_decode_paged(*head, *tail)
    return ea.library().attn_decode_paged_rounded(*head, rounding, *tail)


@pytest.mark.parametrize("kw,code", [
    (dict(tab=None), -1), (dict(lens=None), -1), (dict(q=None), -1),
    (dict(B=0), -2), (dict(Hq=6, Hkv=4), -2), (dict(mb=0), -2), (dict(npages=0), -2),
    (dict(d=256), -3), (dict(page=32), -3), (dict(scale=0.0), -3),
    (dict(k=P + 8), -4), (dict(tab=P + 4), -4),
    (dict(ws=None), -5), (dict(wsb=100), -5),
    (dict(B=65536, wsb=1 << 62), -2), (dict(mb=262141, wsb=1 << 62), -2),   # grid limits
])
def test_decode_argument_errors(kw, code):
    assert dec(**kw) == code
    for r in (0, 1, 2):
        assert dec(rounding=r, **kw) == code
        assert app(rounding=r, **kw) == code


def app(rounding=0, kn=P, vn=P, **kw):
    """attn_decode_paged_append with the same arguments as dec()."""
    a = dict(q=P, k=P, v=P, tab=P, lens=P, o=P, lse=P, B=2, Hq=8, Hkv=2, d=128, page=16,
             mb=4, npages=8, scale=0.1, ws=P, wsb=10 ** 6, stream=None)
    a.update(kw)
    return ea.library().attn_decode_paged_append(
        a["q"], kn, vn, a["k"], a["v"], a["tab"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"],
        a["Hkv"], a["d"], a["page"], a["mb"], a["npages"], a["scale"], rounding, a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), -1), (dict(vn=None), -1), (dict(kn=P + 8), -4), (dict(vn=P + 2), -4),
    (dict(rounding=5), -3),
])
def test_append_argument_errors(kw, code):
    assert app(**kw) == code


def test_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    # all checks pass, so the library asks HIP for the device and finds none
    assert fwd() == -7
    assert fwd(d=64) == -7            # head dims 64 and 256 are supported by attn_fwd
    assert fwd(d=256) == -7
    assert dec() == -7
    assert noalloc() == -7
    for r in (0, 1, 2):
        assert fwd(rounding=r) == -7
        assert dec(rounding=r) == -7
        assert app(rounding=r) == -7


def noalloc(**kw):
    """attn_decode_paged_noalloc with the same arguments as dec(), less the
    workspace."""
    a = dict(q=P, k=P, v=P, tab=P, lens=P, o=P, lse=P, B=2, Hq=8, Hkv=2, d=128, page=16,
             mb=4, npages=8, scale=0.1, stream=None)
    a.update(kw)
    return ea.library().attn_decode_paged_noalloc(
        a["q"], a["k"], a["v"], a["tab"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
        a["d"], a["page"], a["mb"], a["npages"], a["scale"], a["stream"])


NOALLOC_LIMIT = 64 << 20


def test_noalloc_limit_matches_the_binding():
    assert ea.NOALLOC_SCRATCH_BYTES == NOALLOC_LIMIT


@pytest.mark.parametrize("kw,code", [
    (dict(tab=None), -1), (dict(q=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(Hq=6, Hkv=4), -2),
    (dict(d=64), -3), (dict(page=32), -3), (dict(scale=float("nan")), -3),
    (dict(k=P + 8), -4), (dict(lse=P + 4), -4),
    (dict(B=64, Hq=32, Hkv=8, mb=256), -5),     # 68.7 MB of partials: beyond the 64 MiB array
])
def test_noalloc_argument_errors(kw, code):
    assert noalloc(**kw) == code


def test_noalloc_size_limit_edge():
    """The largest problem of a family that fits the array is accepted (up to
    the device check), the next one is refused before any HIP call."""
    B, Hq, mb = 1, 32, 256
    while ea.attn_decode_workspace_bytes(B + 1, Hq, mb) <= NOALLOC_LIMIT:
        B += 1
    assert ea.attn_decode_workspace_bytes(B, Hq, mb) <= NOALLOC_LIMIT
    assert noalloc(B=B + 1, Hq=Hq, Hkv=8, mb=mb) == -5
    import torch
    if not torch.cuda.is_available():
        assert noalloc(B=B, Hq=Hq, Hkv=8, mb=mb) == -7    # checks pass; no device here


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8,
             d=128, scale=0.1, causal=0, layout=0, ws=P, wsb=10 ** 6, stream=None)
    a.update(kw)
    return ea.library().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                 a["d"], a["scale"], a["causal"], a["layout"], a["ws"], a["wsb"],
                                 a["stream"])


def test_bwd_workspace_bytes():
    assert ea.attn_bwd_workspace_bytes(4, 32, 4096) == 8 * 4 * 32 * 4096
    assert ea.attn_bwd_workspace_bytes(1, 1, 1) == 8
    assert ea.attn_bwd_workspace_bytes(0, 1, 1) == 0
    assert ea.attn_bwd_workspace_bytes(1, 1, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(do=None), -1),
    (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(B=0), -2), (dict(Sq=0), -2), (dict(Sk=-1), -2), (dict(Hq=3, Hkv=2), -2),
    (dict(B=65536), -2),
    (dict(Sk=(1 << 22), Hkv=2, Hq=2, layout=0), -2),   # K/V rows of one head exceed 32-bit offsets
    (dict(Sq=(1 << 22), Hkv=2, Hq=2, layout=0, wsb=1 << 40), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(layout=2), -3), (dict(causal=2), -3), (dict(scale=0.0), -3),
    (dict(scale=float("nan")), -3),
    (dict(q=P + 8), -4), (dict(dk=P + 2), -4), (dict(lse=P + 4), -4), (dict(do=P + 8), -4),
    (dict(ws=None), -5), (dict(wsb=8 * 4 * 8 - 1), -5), (dict(ws=P + 4), -5),
])
def test_bwd_argument_errors(kw, code):
    assert bwd(**kw) == code


def test_bwd_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert bwd() == -7
    assert bwd(d=64) == -7            # head dim 64 is supported by attn_bwd


def fwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=3, Hq=4, Hkv=2, tq=100, tk=90, maxq=50,
             d=128, scale=0.1, causal=1, rounding=0, stream=None)
    a.update(kw)
    return ea.library().attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"],
                                        a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"],
                                        a["maxq"], a["d"], a["scale"], a["causal"],
                                        a["rounding"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(cq=None), -1), (dict(ck=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(tq=0), -2), (dict(tk=0), -2), (dict(maxq=0), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(tk=(1 << 21) + 2, Hkv=4), -2),
    # groups of 4k query heads launch 64-row query tiles: B * Hq * ceil(maxq / 64) >= 2^31
    (dict(B=1024, Hq=8, Hkv=2, maxq=1 << 25), -2),
    (dict(d=64), -3), (dict(causal=2), -3), (dict(scale=0.0), -3), (dict(rounding=3), -3),
    (dict(q=P + 8), -4), (dict(o=P + 2), -4), (dict(cq=P + 2), -4), (dict(ck=P + 1), -4),
])
def test_fwd_varlen_argument_errors(kw, code):
    assert fwd_varlen(**kw) == code


def test_fwd_varlen_launch_limit_follows_the_group_size():
    """The same sizes with groups of 2 (256-row query tiles) stay within the
    launch limit and fail only for want of a device."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; valid arguments would launch")
    assert fwd_varlen(B=1024, Hq=8, Hkv=4, maxq=1 << 25) == -7


def test_fwd_varlen_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert fwd_varlen() == -7
    assert fwd_varlen(cq=P + 4, ck=P + 8) == -7   # 4-byte alignment is enough for offsets


def bwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cq=P, ck=P, B=3, Hq=4, Hkv=2,
             tq=100, tk=90, mq=50, mk=60, d=128, scale=0.1, causal=1, ws=P, wsb=10 ** 6,
             stream=None)
    a.update(kw)
    return ea.library().attn_bwd_varlen(
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["cq"],
        a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"], a["d"], a["scale"],
        a["causal"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(cq=None), -1), (dict(ck=None), -1), (dict(dv=None), -1),
    (dict(B=0), -2), (dict(tq=0), -2), (dict(tk=0), -2), (dict(mq=0), -2), (dict(mk=0), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(tk=(1 << 21), Hkv=4), -2),
    (dict(d=64), -3), (dict(causal=2), -3), (dict(scale=-1.0), -3),
    (dict(q=P + 8), -4), (dict(dk=P + 2), -4), (dict(cq=P + 2), -4),
    (dict(ws=None), -5), (dict(wsb=8 * 4 * 100 - 1), -5),
])
def test_bwd_varlen_argument_errors(kw, code):
    assert bwd_varlen(**kw) == code


def test_bwd_varlen_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert bwd_varlen() == -7
    assert bwd_varlen(wsb=8 * 4 * 100) == -7


def fwd_alibi(al=P, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1,
             causal=0, layout=0, rounding=0, stream=None)
    a.update(kw)
    return ea.library().attn_fwd_alibi(a["q"], a["k"], a["v"], a["o"], a["lse"], al, a["B"],
                                       a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"],
                                       a["causal"], a["layout"], a["rounding"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(al=None), -1), (dict(q=None), -1), (dict(al=P + 2), -4), (dict(B=0), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(d=64), -3), (dict(rounding=9), -3), (dict(o=P + 8), -4),
    (dict(d=96), -3),
])
def test_fwd_alibi_argument_errors(kw, code):
    assert fwd_alibi(**kw) == code


def test_fwd_alibi_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert fwd_alibi() == -7
    assert fwd_alibi(al=P + 4) == -7


def bwd_alibi(al=P, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8,
             d=128, scale=0.1, causal=0, layout=0, ws=P, wsb=10 ** 6, stream=None)
    a.update(kw)
    return ea.library().attn_bwd_alibi(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                                       a["dq"], a["dk"], a["dv"], al, a["B"], a["Hq"], a["Hkv"],
                                       a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"],
                                       a["layout"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(al=None), -1), (dict(dq=None), -1), (dict(al=P + 2), -4), (dict(B=0), -2),
    (dict(d=64), -3), (dict(ws=None), -5),
])
def test_bwd_alibi_argument_errors(kw, code):
    assert bwd_alibi(**kw) == code


def test_binding_rejects_unknown_rounding_name():
    with pytest.raises(ValueError):
        ea._rounding_code("nearest")
    assert [ea._rounding_code(n) for n in ("RTNE", "rtna", "rtz")] == [0, 1, 2]


def fwd_fp8(**kw):
    a = dict(q=P, k=P, v=P, dq=1.0, dk=1.0, dv=1.0, o=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8,
             d=128, scale=0.1, causal=0, layout=0, stream=None)
    a.update(kw)
    return ea.library().attn_fwd_fp8(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"],
                                     a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                                     a["scale"], a["causal"], a["layout"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(B=0), -2), (dict(Hq=3), -2), (dict(Sk=0), -2),
    (dict(d=64), -3), (dict(layout=2), -3), (dict(causal=2), -3), (dict(dq=0.0), -3),
    (dict(dk=-1.0), -3), (dict(dv=float("inf")), -3), (dict(dv=float("nan")), -3),
    (dict(dq=1e-30, dk=1e-30), -3), (dict(dq=1e30, dk=1e30), -3), (dict(v=P + 8), -4),
    (dict(Sk=1 << 24, Hq=2, Hkv=1), -2),    # K/V head beyond 32-bit byte offsets
])
def test_fwd_fp8_argument_errors(kw, code):
    assert fwd_fp8(**kw) == code


def test_fwd_fp8_valid_arguments_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert fwd_fp8() == -7
    assert fwd_fp8(dq=0.5, dk=3.0, dv=1e-3, causal=1, layout=1) == -7
