"""Exact attention on MI355X (gfx950): Python binding of libattn.so.

The binding only marshals arguments: it checks tensor dtypes, devices and
shapes, allocates outputs (and the decode workspace) with torch, and calls the
C ABI declared in include/attn.h with raw pointers and the current HIP stream.
Every step of the computation runs in the library's HIP kernels; if the
library is not built the binding raises instead of computing anything itself.

    o, lse = attn_fwd(q, k, v, causal=False, scale=None, layout="bshd", rounding="rtne")
    o, lse = attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, rounding="rtne")
    o, lse = attn_decode_paged_append(q, k_new, v_new, k_cache, v_cache, block_table,
                                      seq_lens)   # writes the new rows into the caches
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=False, scale=None, layout="bshd")
    o, lse = attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q)  # packed
    dq, dk, dv = attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k,
                                 max_seqlen_q, max_seqlen_k)

``rounding`` is the rule of the final fp32 -> bf16 conversion of O: "rtne"
(nearest, ties to even; the plain entry points), "rtna" (nearest, ties away
from zero) or "rtz" (toward zero); the other two call the *_rounded entry
points.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_BSHD = 0
ATTN_BHSD = 1
HEAD_DIM = 128
PAGE_SIZE = 16
ROUNDING = {"rtne": 0, "rtna": 1, "rtz": 2}

STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_UNSUPPORTED",
    -4: "ATTN_ERR_ALIGN", -5: "ATTN_ERR_WORKSPACE", -6: "ATTN_ERR_LAUNCH",
    -7: "ATTN_ERR_DEVICE",
}

# every symbol include/attn.h declares
EXPORTS = ("attn_fwd", "attn_fwd_rounded", "attn_prep_v_bytes", "attn_prep_v", "attn_fwd_prepped",
           "attn_fwd_alibi", "attn_fwd_varlen", "attn_fwd_fp8",
           "attn_decode_workspace_bytes", "attn_decode_paged",
           "attn_decode_paged_rounded", "attn_decode_paged_append", "attn_decode_paged_noalloc",
           "attn_bwd_workspace_bytes",
           "attn_bwd", "attn_bwd_alibi", "attn_bwd_varlen", "attn_status_string", "attn_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = library().attn_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def library() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by exact_attention_60_amd._build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m exact_attention_60_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        lib.attn_fwd.restype = i
        lib.attn_fwd_rounded.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
        lib.attn_fwd_rounded.restype = i
        lib.attn_prep_v_bytes.argtypes = [i, i, i, i, i]
        lib.attn_prep_v_bytes.restype = sz
        lib.attn_prep_v.argtypes = [vp, i, i, i, i, i, i, vp, sz, vp]
        lib.attn_prep_v.restype = i
        lib.attn_fwd_prepped.argtypes = [vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, f, i, i, i,
                                         vp]
        lib.attn_fwd_prepped.restype = i
        lib.attn_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
        lib.attn_fwd_alibi.restype = i
        lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i,
                                        vp]
        lib.attn_fwd_varlen.restype = i
        lib.attn_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        lib.attn_fwd_fp8.restype = i
        lib.attn_decode_workspace_bytes.argtypes = [i, i, i]
        lib.attn_decode_workspace_bytes.restype = sz
        lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp,
                                          sz, vp]
        lib.attn_decode_paged.restype = i
        lib.attn_decode_paged_rounded.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                                  f, i, vp, sz, vp]
        lib.attn_decode_paged_rounded.restype = i
        lib.attn_decode_paged_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i,
                                                 i, i, i, f, i, vp, sz, vp]
        lib.attn_decode_paged_append.restype = i
        lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                                  f, vp]
        lib.attn_decode_paged_noalloc.restype = i
        lib.attn_bwd_workspace_bytes.argtypes = [i, i, i]
        lib.attn_bwd_workspace_bytes.restype = sz
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp,
                                 sz, vp]
        lib.attn_bwd.restype = i
        lib.attn_bwd_alibi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f,
                                       i, i, vp, sz, vp]
        lib.attn_bwd_alibi.restype = i
        lib.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                        i, i, i, f, i, vp, sz, vp]
        lib.attn_bwd_varlen.restype = i
        lib.attn_status_string.argtypes = [i]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_version.argtypes = []
        lib.attn_version.restype = i
        _lib = lib
    return _lib


def attn_version() -> int:
    return library().attn_version()


def attn_status_string(status: int) -> str:
    return library().attn_status_string(status).decode()


def attn_decode_workspace_bytes(B: int, Hq: int, max_blocks_per_seq: int) -> int:
    return int(library().attn_decode_workspace_bytes(B, Hq, max_blocks_per_seq))


def attn_bwd_workspace_bytes(B: int, Hq: int, Sq: int) -> int:
    return int(library().attn_bwd_workspace_bytes(B, Hq, Sq))


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_bf16(name, t):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(name, t, dtype, shape, device):
    """A caller-supplied output (or workspace) must match what the kernels
    write: dtype, exact shape, the inputs' device, contiguous."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_same_device(dev, **tensors):
    for n, t in tensors.items():
        if t.device != dev:
            raise ValueError(f"{n} must be on {dev} (the device of q), got {t.device}")


def _workspace(ws, need, device):
    """The caller's workspace (a contiguous GPU byte tensor of at least `need`
    bytes) or a fresh one."""
    torch = _torch()
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")
    return ws


def _rounding_code(rounding: str) -> int:
    try:
        return ROUNDING[rounding.lower()]
    except KeyError:
        raise ValueError(f"rounding must be one of {sorted(ROUNDING)}, got {rounding!r}") from None


# query tiles (256 rows) per K/V head from which attn_fwd prepares V by default
PREPARE_V_MIN_TILES = 32
PREPARE_V_MIN_BLOCKS_D256 = 16
PREPARE_V_MIN_BLOCKS_D64 = 32


def attn_prep_v_bytes(B: int, Hq: int, Hkv: int, Sk: int, d: int) -> int:
    return library().attn_prep_v_bytes(B, Hq, Hkv, Sk, d)


def prepares_v(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int) -> bool:
    """Whether attn_fwd (no ALiBi, prepare_v=None) runs attn_prep_v +
    attn_fwd_prepped for this shape: at d = 128 when each K/V head serves at
    least PREPARE_V_MIN_TILES query tiles of 256 rows, at d = 256 and d = 64
    at least PREPARE_V_MIN_BLOCKS_D256 / PREPARE_V_MIN_BLOCKS_D64 query blocks
    of 128 rows (Sq * Hq / Hkv rows per K/V head)."""
    rows = Sq * (Hq // Hkv)
    if d == 256:
        many = (rows + 127) // 128 >= PREPARE_V_MIN_BLOCKS_D256
    elif d == 64:
        many = (rows + 127) // 128 >= PREPARE_V_MIN_BLOCKS_D64
    else:
        many = (rows + 255) // 256 >= PREPARE_V_MIN_TILES
    return many and attn_prep_v_bytes(B, Hq, Hkv, Sk, d) > 0


def attn_fwd(q, k, v, *, causal: bool = False, scale: float | None = None,
             layout: str = "bshd", rounding: str = "rtne", out=None, lse=None, stream=None,
             alibi_slopes=None, prepare_v: bool | None = None, vt=None):
    """Fused exact attention forward.  q: [B, Sq, Hq, d] (bshd) or
    [B, Hq, Sq, d] (bhsd); k, v likewise with Hkv heads and Sk keys.  The head
    dim d is 128, 64 or 256 (64 and 256 without ALiBi).
    alibi_slopes: optional fp32 GPU tensor [Hq] (ALiBi bias, attn_fwd_alibi).
    prepare_v: where the shape uses prepared fp16 V^T tiles
    (attn_prep_v_bytes > 0, no ALiBi), True runs attn_prep_v into `vt` (a
    uint8 GPU tensor of at least that many bytes, allocated here if None) and
    then attn_fwd_prepped; False runs the single-call attn_fwd /
    attn_fwd_rounded.  None (default) follows prepares_v: the one conversion
    per head costs less than the per-workgroup ones it replaces once each K/V
    head serves enough query rows (measured at d = 128: even at 16 tiles of
    256 rows, MHA B=4 H=32 S=4096, both 1023-1043 TFLOP/s; +2 % at 32 tiles,
    a gain at 128; at d = 256: a loss at 8 blocks of 128 rows, a
    gain at 32; at d = 64: a loss at 8, even at 64 on a short causal shape, a
    gain of 4-6 % at 32 and 256).
    Returns (o bf16 in q's layout, lse fp32 [B, Hq, Sq])."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be 4-D and k, v of equal shape")
    lay = {"bshd": ATTN_BSHD, "bhsd": ATTN_BHSD}[layout.lower()]
    rnd = _rounding_code(rounding)
    if lay == ATTN_BSHD:
        B, Sq, Hq, d = q.shape
        _, Sk, Hkv, _ = k.shape
    else:
        B, Hq, Sq, d = q.shape
        _, Hkv, Sk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q and k disagree on batch or head dim")
    _check_same_device(q.device, k=k, v=v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, torch.float32, (B, Hq, Sq), q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
            Sq, Sk, d, float(scale), int(bool(causal)), lay)
    if alibi_slopes is not None:
        _check_out("alibi_slopes", alibi_slopes, torch.float32, (Hq,), q.device)
        st = library().attn_fwd_alibi(*args[:5], alibi_slopes.data_ptr(), *args[5:], rnd,
                                      _stream_ptr(stream))
        where = "attn_fwd_alibi"
    elif (prepare_v if prepare_v is not None else prepares_v(B, Hq, Hkv, Sq, Sk, d)) and \
            (nvt := library().attn_prep_v_bytes(B, Hq, Hkv, Sk, d)) > 0:
        vt = _workspace(vt, nvt, q.device)
        nb = vt.numel() * vt.element_size()
        st = library().attn_prep_v(v.data_ptr(), B, Hq, Hkv, Sk, d, lay, vt.data_ptr(), nb,
                                   _stream_ptr(stream))
        where = "attn_prep_v"
        if st == 0:
            st = library().attn_fwd_prepped(*args[:3], vt.data_ptr(), nb, *args[3:], rnd,
                                            _stream_ptr(stream))
            where = "attn_fwd_prepped"
    elif rnd == ROUNDING["rtne"]:
        st, where = library().attn_fwd(*args, _stream_ptr(stream)), "attn_fwd"
    else:
        st, where = library().attn_fwd_rounded(*args, rnd, _stream_ptr(stream)), "attn_fwd_rounded"
    if st != 0:
        raise AttnError(st, where)
    return out, lse


def attn_fwd_fp8(q, k, v, *, descale_q: float = 1.0, descale_k: float = 1.0,
                 descale_v: float = 1.0, causal: bool = False, scale: float | None = None,
                 layout: str = "bshd", out=None, lse=None, stream=None):
    """Attention forward on FP8 inputs: q, k, v are uint8 GPU tensors of OCP
    E4M3 bytes (or torch.float8_e4m3fn), shaped as for attn_fwd, each with a
    per-tensor fp32 descale.  Returns (o bf16 in q's layout, lse fp32
    [B, Hq, Sq])."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_cuda or \
                not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous uint8 / float8_e4m3fn GPU tensor")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be 4-D and k, v of equal shape")
    lay = {"bshd": ATTN_BSHD, "bhsd": ATTN_BHSD}[layout.lower()]
    if lay == ATTN_BSHD:
        B, Sq, Hq, d = q.shape
        _, Sk, Hkv, _ = k.shape
    else:
        B, Hq, Sq, d = q.shape
        _, Hkv, Sk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q and k disagree on batch or head dim")
    _check_same_device(q.device, k=k, v=v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check_out("out", out, torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, torch.float32, (B, Hq, Sq), q.device)
    st = library().attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(descale_q),
                                float(descale_k), float(descale_v), out.data_ptr(), lse.data_ptr(),
                                B, Hq, Hkv, Sq, Sk, d, float(scale), int(bool(causal)), lay,
                                _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, *,
                    causal: bool = False, scale: float | None = None, rounding: str = "rtne",
                    out=None, lse=None, stream=None):
    """Attention forward over packed sequences.  q: [total_q, Hq, 128];
    k, v: [total_k, Hkv, 128]; cu_seqlens_q / cu_seqlens_k: int32 GPU tensors
    [B + 1] of row offsets; max_seqlen_q: the longest query length (a host
    int).  Returns (o bf16 [total_q, Hq, 128], lse fp32 [Hq, total_q])."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t)
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{n} must be a contiguous 1-D int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    _check_same_device(q.device, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, torch.float32, (Hq, total_q), q.device)
    st = library().attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), cu_seqlens_q.data_ptr(),
                                   cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k,
                                   int(max_seqlen_q), d, float(scale), int(bool(causal)),
                                   _rounding_code(rounding), _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_varlen")
    return out, lse


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, scale: float | None = None,
                      rounding: str = "rtne", out=None, lse=None, workspace=None, stream=None,
                      k_new=None, v_new=None):
    """One paged decode step.  q: [B, Hq, 128]; k_cache, v_cache:
    [num_pages, 16, Hkv, 128]; block_table: int32 [B, max_blocks];
    seq_lens: int32 [B].  Returns (o bf16 [B, Hq, 128], lse fp32 [B, Hq])."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(n, t)
    append = k_new is not None or v_new is not None
    if append:
        if k_new is None or v_new is None:
            raise ValueError("k_new and v_new go together")
        _check_bf16("k_new", k_new)
        _check_bf16("v_new", v_new)
    for n, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q must be [B, Hq, d], the caches [num_pages, 16, Hkv, d], "
                         "block_table [B, max_blocks] and seq_lens [B]")
    B, Hq, d = q.shape
    num_pages, page, Hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or block_table.shape[0] != B:
        raise ValueError("inconsistent decode shapes")
    if seq_lens.numel() != B:
        raise ValueError(f"seq_lens must hold B = {B} lengths, got {seq_lens.numel()}")
    _check_same_device(q.device, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                       seq_lens=seq_lens)
    if append:
        _check_same_device(q.device, k_new=k_new, v_new=v_new)
    if append and (tuple(k_new.shape) != (B, Hkv, d) or tuple(v_new.shape) != (B, Hkv, d)):
        raise ValueError("k_new and v_new must be [B, Hkv, 128]")
    max_blocks = block_table.shape[1]
    rnd = _rounding_code(rounding)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_decode_workspace_bytes(B, Hq, max_blocks)
    workspace = _workspace(workspace, need, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, torch.float32, (B, Hq), q.device)
    head = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
            seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, page, max_blocks,
            num_pages, float(scale))
    tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if append:
        st = library().attn_decode_paged_append(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), *head[1:], rnd, *tail)
        where = "attn_decode_paged_append"
    elif rnd == ROUNDING["rtne"]:
        st, where = library().attn_decode_paged(*head, *tail), "attn_decode_paged"
    else:
        st, where = library().attn_decode_paged_rounded(*head, rnd, *tail), "attn_decode_paged_rounded"
    if st != 0:
        raise AttnError(st, where)
    return out, lse


# bytes of the device scratch array attn_decode_paged_noalloc uses (per GPU)
NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *,
                              scale: float | None = None, out=None, lse=None, stream=None):
    """attn_decode_paged (RTNE) through the entry point that allocates
    nothing: the split partials use the library's own device scratch array
    (NOALLOC_SCRATCH_BYTES per GPU; larger problems raise).  Pass out and lse
    to allocate nothing here either.  Calls that overlap on one GPU race."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(n, t)
    for n, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q must be [B, Hq, d], the caches [num_pages, 16, Hkv, d], "
                         "block_table [B, max_blocks] and seq_lens [B]")
    B, Hq, d = q.shape
    num_pages, page, Hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or block_table.shape[0] != B or \
            seq_lens.numel() != B:
        raise ValueError("inconsistent decode shapes")
    _check_same_device(q.device, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                       seq_lens=seq_lens)
    max_blocks = block_table.shape[1]
    if attn_decode_workspace_bytes(B, Hq, max_blocks) > NOALLOC_SCRATCH_BYTES:
        raise ValueError("problem too large for the no-allocation decode's scratch array")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, torch.float32, (B, Hq), q.device)
    st = library().attn_decode_paged_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, page, max_blocks,
        num_pages, float(scale), _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_noalloc")
    return out, lse


def attn_decode_paged_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, **kw):
    """Append the current token (K/V rows k_new, v_new: [B, Hkv, 128]) to the
    paged caches at position seq_lens[b] - 1, then decode over every token;
    the caches are written in place.  Returns (o, lse)."""
    return attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, k_new=k_new,
                             v_new=v_new, **kw)


def attn_bwd(q, k, v, o, lse, do, *, causal: bool = False, scale: float | None = None,
             layout: str = "bshd", dq=None, dk=None, dv=None, workspace=None, stream=None,
             alibi_slopes=None):
    """Gradients of attn_fwd (head dim 128, or 64 without ALiBi) for an
    upstream gradient do (q's layout and shape), from the forward's inputs q, k, v and outputs o, lse (and its
    ALiBi slopes, if it had any: attn_bwd_alibi).  Returns (dq in q's layout,
    dk and dv in k's layout), all bf16."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_bf16(n, t)
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4 or o.shape != q.shape or \
            do.shape != q.shape:
        raise ValueError("q, o, do must share a 4-D shape and k, v another")
    lay = {"bshd": ATTN_BSHD, "bhsd": ATTN_BHSD}[layout.lower()]
    if lay == ATTN_BSHD:
        B, Sq, Hq, d = q.shape
        _, Sk, Hkv, _ = k.shape
    else:
        B, Hq, Sq, d = q.shape
        _, Hkv, Sk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q and k disagree on batch or head dim")
    _check_same_device(q.device, k=k, v=v, o=o, do=do)
    _check_out("lse", lse, torch.float32, (B, Hq, Sq), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_out("dq", dq, torch.bfloat16, q.shape, q.device)
    _check_out("dk", dk, torch.bfloat16, k.shape, q.device)
    _check_out("dv", dv, torch.bfloat16, v.shape, q.device)
    need = attn_bwd_workspace_bytes(B, Hq, Sq)
    workspace = _workspace(workspace, need, q.device)
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    tail = (B, Hq, Hkv, Sq, Sk, d, float(scale), int(bool(causal)), lay, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if alibi_slopes is not None:
        _check_out("alibi_slopes", alibi_slopes, torch.float32, (Hq,), q.device)
        st, where = library().attn_bwd_alibi(*head, alibi_slopes.data_ptr(), *tail), "attn_bwd_alibi"
    else:
        st, where = library().attn_bwd(*head, *tail), "attn_bwd"
    if st != 0:
        raise AttnError(st, where)
    return dq, dk, dv


def attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    max_seqlen_k: int, *, causal: bool = False, scale: float | None = None,
                    dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of attn_fwd_varlen for an upstream gradient do
    ([total_q, Hq, 128]), from its inputs and its outputs o, lse
    ([Hq, total_q]).  Returns (dq, dk, dv) in the packed layouts, bf16."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_bf16(n, t)
    if q.dim() != 3 or k.shape != v.shape or k.dim() != 3 or o.shape != q.shape or \
            do.shape != q.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q, o, do must share a [total_q, Hq, d] shape and k, v [total_k, Hkv, d]")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{n} must be a contiguous 1-D int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    _check_same_device(q.device, k=k, v=v, o=o, do=do, cu_seqlens_q=cu_seqlens_q,
                       cu_seqlens_k=cu_seqlens_k)
    _check_out("lse", lse, torch.float32, (Hq, total_q), q.device)
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_out("dq", dq, torch.bfloat16, q.shape, q.device)
    _check_out("dk", dk, torch.bfloat16, k.shape, q.device)
    _check_out("dv", dv, torch.bfloat16, v.shape, q.device)
    need = attn_bwd_workspace_bytes(1, Hq, total_q)
    workspace = _workspace(workspace, need, q.device)
    st = library().attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), cu_seqlens_q.data_ptr(),
                                   cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k,
                                   int(max_seqlen_q), int(max_seqlen_k), d, float(scale),
                                   int(bool(causal)), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_varlen")
    return dq, dk, dv


__all__ = ["attn_fwd", "attn_fwd_varlen", "attn_bwd", "attn_bwd_varlen", "attn_bwd_workspace_bytes", "attn_decode_paged", "attn_decode_paged_append", "attn_decode_paged_noalloc", "NOALLOC_SCRATCH_BYTES",
           "attn_decode_workspace_bytes", "attn_status_string",
           "attn_version", "attn_prep_v_bytes", "prepares_v", "PREPARE_V_MIN_TILES",
           "PREPARE_V_MIN_BLOCKS_D256", "PREPARE_V_MIN_BLOCKS_D64", "library", "AttnError", "ATTN_BSHD", "ATTN_BHSD", "ROUNDING", "EXPORTS",
           "LIB_PATH"]
