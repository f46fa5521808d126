"""Seeded synthetic inputs for the attention forward and the paged decode.

This module only draws and encodes data: it holds none of the attention
arithmetic.  Both the HIP path (through the binding) and the CPU oracle take
their inputs from here, and from nowhere else.

Every array is drawn in float32 from NumPy's PCG64 generator seeded with
``[seed, stream_id]`` and rounded to bfloat16 (round to nearest, ties to even)
by bit arithmetic.  bf16 tensors are returned as ``uint16`` arrays of their bit
patterns, in the memory layout the library consumes:

* BSHD: ``[B, S, H, D]``; BHSD: ``[B, H, S, D]`` (D innermost in both).
* Paged KV pool: ``[num_pages, 16, Hkv, D]`` with an int32 block table
  ``[B, max_blocks]`` (unused entries are -1) and int32 ``seq_lens``.

The five named workloads below are synthetic stand-ins for the workloads the
pages measure on (Llama-style GQA prefill, video-diffusion self and cross
attention, vLLM-style paged decode): same shapes, value distributions and
structure, random data.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D = 128
PAGE = 16
BF16_QNAN = np.uint16(0x7FC0)

# stream ids for default_rng([seed, stream])
(_S_Q, _S_K, _S_V, _S_HOT, _S_LENS, _S_PERM, _S_KX, _S_VX, _S_EQK, _S_EQV, _S_KNEW,
 _S_VNEW, _S_DO, _S_VLENS, _S_F8Q, _S_F8K, _S_F8V) = range(17)

BSHD = 0
BHSD = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def _normal(seed, stream, shape):
    return _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)


def _uniform(seed, stream, shape, lo=-1.0, hi=1.0):
    return _rng(seed, stream).uniform(lo, hi, size=shape).astype(np.float32)


def _draw(dist, seed, stream, shape):
    if dist == "normal":
        return _normal(seed, stream, shape)
    if dist == "uniform":
        return _uniform(seed, stream, shape)
    if dist == "zeros":
        return np.zeros(shape, np.float32)
    raise ValueError(dist)


def layout_shape(layout: int, B: int, H: int, S: int, d: int = D):
    return (B, S, H, d) if layout == BSHD else (B, H, S, d)


@dataclass
class Prefill:
    """One prefill problem; q/k/v are bf16 bit arrays in `layout`."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    layout: int
    causal: bool
    scale: float
    name: str = ""
    hot_rows: list = field(default_factory=list)  # (b, s, h) query vectors scaled x8

    @property
    def d(self) -> int:
        return int(self.q.shape[-1])

    @property
    def flops(self) -> float:
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * self.d
        return f / 2 if self.causal else f


def prefill_inputs(B, Hq, Hkv, Sq, Sk, *, layout=BSHD, causal=False, seed=0,
                   scale=None, q_dist="normal", k_dist="normal", v_dist="normal",
                   n_hot=0, name="", d=D, v_amp=1.0) -> Prefill:
    """Draw a prefill problem (head dim d, 128 unless given).  `n_hot` query
    vectors Q[b, s, h, :] (drawn by the seed) are multiplied by 8 before
    rounding; x8 is a power of two, so it commutes with the bf16 rounding.
    V's draws are multiplied by v_amp (in float32) before rounding."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qf = _draw(q_dist, seed, _S_Q, layout_shape(layout, B, Hq, Sq, d))
    hot = []
    if n_hot:
        r = _rng(seed, _S_HOT)
        flat = r.choice(B * Sq * Hq, size=n_hot, replace=False)
        for f in sorted(int(x) for x in flat):
            b, rem = divmod(f, Sq * Hq)
            s, h = divmod(rem, Hq)
            hot.append((b, s, h))
            if layout == BSHD:
                qf[b, s, h, :] *= 8.0
            else:
                qf[b, h, s, :] *= 8.0
    q = f32_to_bf16_bits(qf)
    del qf
    k = f32_to_bf16_bits(_draw(k_dist, seed, _S_K, layout_shape(layout, B, Hkv, Sk, d)))
    v = f32_to_bf16_bits(np.float32(v_amp) *
                         _draw(v_dist, seed, _S_V, layout_shape(layout, B, Hkv, Sk, d)))
    return Prefill(q, k, v, B, Hq, Hkv, Sq, Sk, layout, bool(causal), float(scale),
                   name=name, hot_rows=hot)


@dataclass
class Decode:
    q: np.ndarray            # bf16 bits [B, Hq, D]
    k_pool: np.ndarray       # bf16 bits [P, 16, Hkv, D]
    v_pool: np.ndarray
    block_table: np.ndarray  # int32 [B, max_blocks], -1 beyond each sequence
    seq_lens: np.ndarray     # int32 [B]
    B: int
    Hq: int
    Hkv: int
    scale: float
    name: str = ""

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: K and V of every valid token of every KV
        head, plus Q, O, LSE, the block-table entries read and seq_lens."""
        n_pages_read = int(sum((int(x) + PAGE - 1) // PAGE for x in self.seq_lens))
        return (2 * D * 2 * self.Hkv * self.tokens + self.B * self.Hq * D * 2 * 2
                + self.B * self.Hq * 4 + n_pages_read * 4 + self.B * 4)

    @property
    def flops(self) -> float:
        return 4.0 * self.Hq * D * self.tokens


def decode_inputs(B, Hq, Hkv, *, max_len=4096, seed=0, scale=None, lens=None,
                  permute=True, poison_tail=True, name="", q_amp=1.0, v_amp=1.0) -> Decode:
    """Paged decode problem: lens ~ U{1..max_len} (unless given), 16-token
    pages dealt out in sequence order from one random permutation of the pool;
    slots past each sequence's end hold bf16 NaN.  Q's and V's draws are
    multiplied by q_amp and v_amp (in float32) before rounding."""
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if lens is None:
        lens = _rng(seed, _S_LENS).integers(1, max_len + 1, size=B)
    lens = np.asarray(lens, dtype=np.int32)
    assert lens.shape == (B,) and lens.min() >= 1
    max_blocks = (max_len + PAGE - 1) // PAGE
    nb = (lens.astype(np.int64) + PAGE - 1) // PAGE
    assert nb.max() <= max_blocks
    P = int(nb.sum())
    ids = _rng(seed, _S_PERM).permutation(P) if permute else np.arange(P)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nb[b]] = ids[off:off + nb[b]]
        off += int(nb[b])
    kp = f32_to_bf16_bits(_normal(seed, _S_K, (P, PAGE, Hkv, D)))
    vp = f32_to_bf16_bits(np.float32(v_amp) * _normal(seed, _S_V, (P, PAGE, Hkv, D)))
    if poison_tail:
        for b in range(B):
            t = int(lens[b]) % PAGE
            if t:
                last = table[b, nb[b] - 1]
                kp[last, t:] = BF16_QNAN
                vp[last, t:] = BF16_QNAN
    q = f32_to_bf16_bits(np.float32(q_amp) * _normal(seed, _S_Q, (B, Hq, D)))
    return Decode(q, kp, vp, table, lens, B, Hq, Hkv, float(scale), name=name)


@dataclass
class DecodeAppend:
    """A decode step that first appends the current token: `base` is the
    paged problem (lengths count the current token), k_new / v_new its K and V
    rows (bf16 bits [B, Hkv, D]).  The pool slots of the current tokens hold
    bf16 NaN, standing for cache memory not yet written."""
    base: Decode
    k_new: np.ndarray
    v_new: np.ndarray


def decode_append_inputs(B, Hq, Hkv, *, max_len=4096, seed=0, lens=None, name="") -> DecodeAppend:
    d = decode_inputs(B, Hq, Hkv, max_len=max_len, seed=seed, lens=lens, name=name)
    for b in range(B):
        t = int(d.seq_lens[b]) - 1
        page = d.block_table[b, t // PAGE]
        d.k_pool[page, t % PAGE] = BF16_QNAN
        d.v_pool[page, t % PAGE] = BF16_QNAN
    k_new = f32_to_bf16_bits(_normal(seed, _S_KNEW, (B, Hkv, D)))
    v_new = f32_to_bf16_bits(_normal(seed, _S_VNEW, (B, Hkv, D)))
    return DecodeAppend(d, k_new, v_new)


# --------------------------------------------------------------------------
# Structured inputs for exactness checks: every key of a (sequence, K/V head)
# is one random vector, so all visible scores of a query row are equal, and V
# holds values with few significant bits, so that sums of a few of them are
# exact in float32.

def short_values(seed, stream, shape, binades=0) -> np.ndarray:
    """bf16 bits of s * (1 + m/128) * 2^e with a random sign s, m ~ U{0..127}
    and e ~ U{-binades..binades}: every bf16 significand in 2*binades + 1
    binades."""
    r = _rng(seed, stream)
    m = r.integers(0, 128, size=shape).astype(np.uint32)
    e = r.integers(-binades, binades + 1, size=shape).astype(np.int64)
    sign = r.integers(0, 2, size=shape).astype(np.uint32)
    bits = (sign << 15) | ((127 + e).astype(np.uint32) << 7) | m
    return bits.astype(np.uint16)


def equal_keys_prefill(B, Hq, Hkv, Sq, Sk, *, layout=BSHD, causal=False, seed=0,
                       binades=0, name="") -> Prefill:
    """Q ~ N(0, 1); K[b, :, g] is one N(0, 1) vector repeated over the keys;
    V from short_values."""
    q = f32_to_bf16_bits(_normal(seed, _S_Q, layout_shape(layout, B, Hq, Sq)))
    row = f32_to_bf16_bits(_normal(seed, _S_EQK, (B, 1, Hkv, D)))
    k = np.ascontiguousarray(np.broadcast_to(row, (B, Sk, Hkv, D)))
    v = short_values(seed, _S_EQV, (B, Sk, Hkv, D), binades)
    if layout == BHSD:
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    return Prefill(q, k, v, B, Hq, Hkv, Sq, Sk, layout, bool(causal), 1.0 / math.sqrt(D),
                   name=name)


def equal_keys_decode(lens, Hq, Hkv, *, seed=0, binades=0, name="") -> Decode:
    """A paged problem (decode_inputs, random table) whose K rows are one
    N(0, 1) vector per (sequence, K/V head) and whose V values come from
    short_values; slots past each sequence's end keep the NaN poison."""
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.shape[0]
    max_len = int(-(-int(lens.max()) // PAGE) * PAGE)
    p = decode_inputs(B, Hq, Hkv, max_len=max_len, seed=seed, lens=lens, name=name)
    rows = f32_to_bf16_bits(_normal(seed, _S_EQK, (B, Hkv, D)))
    vals = short_values(seed, _S_EQV, p.v_pool.shape, binades)
    for b in range(B):
        n = int(lens[b])
        for t in range(n):
            pg = p.block_table[b, t // PAGE]
            p.k_pool[pg, t % PAGE] = rows[b]
            p.v_pool[pg, t % PAGE] = vals[pg, t % PAGE]
    return p


def output_grad(p: Prefill, seed=0, dist="normal") -> np.ndarray:
    """Upstream gradient dO for the backward of problem p: bf16 bits in Q's
    layout and shape, iid N(0, 1) by default."""
    return f32_to_bf16_bits(_draw(dist, seed, _S_DO, layout_shape(p.layout, p.B, p.Hq, p.Sq,
                                                               p.d)))


@dataclass
class Varlen:
    """Packed sequences: q [total_q, Hq, D], k/v [total_k, Hkv, D] bf16 bits;
    sequence b is rows cu_q[b]..cu_q[b+1]-1 of q and cu_k[b]..cu_k[b+1]-1 of
    k/v (int32 offsets)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    Hq: int
    Hkv: int
    causal: bool
    scale: float
    name: str = ""

    @property
    def B(self) -> int:
        return len(self.cu_q) - 1

    @property
    def max_q(self) -> int:
        return max(1, int(np.diff(self.cu_q).max()))

    @property
    def flops(self) -> float:
        """4*Hq*Sq_b*Sk_b*D summed over the sequences, halved when causal."""
        f = 4.0 * self.Hq * float(np.sum(np.diff(self.cu_q).astype(np.float64) *
                                         np.diff(self.cu_k))) * D
        return f / 2 if self.causal else f


def varlen_inputs(lens_q, lens_k, Hq, Hkv, *, causal=False, seed=0, name="") -> Varlen:
    """Packed sequences with the given query and key lengths; Q, K, V iid
    N(0, 1)."""
    lens_q = np.asarray(lens_q, np.int64)
    lens_k = np.asarray(lens_k, np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = f32_to_bf16_bits(_normal(seed, _S_Q, (int(cu_q[-1]), Hq, D)))
    k = f32_to_bf16_bits(_normal(seed, _S_K, (int(cu_k[-1]), Hkv, D)))
    v = f32_to_bf16_bits(_normal(seed, _S_V, (int(cu_k[-1]), Hkv, D)))
    return Varlen(q, k, v, cu_q, cu_k, Hq, Hkv, bool(causal), 1.0 / math.sqrt(D), name=name)


# --------------------------------------------------------------------------
# The named workloads (d = 128, bf16, scale = 1/sqrt(128) throughout).

def config1(seed=1):
    """Tiny MHA forward, BSHD, non-causal; 8 query vectors scaled x8."""
    return prefill_inputs(1, 4, 4, 256, 256, layout=BSHD, seed=seed, n_hot=8,
                          name="mha_tiny_b1_h4_s256_bshd")


def config2(seed=2):
    """MHA prefill B=4, H=32, S=4096, BHSD, non-causal."""
    return prefill_inputs(4, 32, 32, 4096, 4096, layout=BHSD, seed=seed,
                          name="mha_prefill_b4_h32_s4096_bhsd")


def config3(seed=3):
    """Causal GQA prefill B=8, Hq=32, Hkv=8, S=8192, BSHD; V ~ U(-1, 1)."""
    return prefill_inputs(8, 32, 8, 8192, 8192, layout=BSHD, causal=True,
                          seed=seed, v_dist="uniform",
                          name="gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd")


def config4_self(seed=4):
    """Diffusion-style self attention B=2, H=12, S=32760, BSHD."""
    return prefill_inputs(2, 12, 12, 32760, 32760, layout=BSHD, seed=seed,
                          name="diffusion_self_b2_h12_s32760_bshd")


def config4_cross(seed=4, self_problem: Prefill | None = None):
    """Cross attention reusing the self-attention Q against 512 fresh keys."""
    if self_problem is None:
        self_problem = config4_self(seed)
    k = f32_to_bf16_bits(_normal(seed, _S_KX, layout_shape(BSHD, 2, 12, 512)))
    v = f32_to_bf16_bits(_normal(seed, _S_VX, layout_shape(BSHD, 2, 12, 512)))
    return Prefill(self_problem.q, k, v, 2, 12, 12, 32760, 512, BSHD, False,
                   self_problem.scale, name="diffusion_cross_b2_h12_sq32760_sk512_bshd")


def config5(seed=5):
    """Paged split-KV decode B=32, Hq=32, Hkv=8, lens ~ U{1..4096}."""
    return decode_inputs(32, 32, 8, max_len=4096, seed=seed,
                         name="paged_decode_b32_hq32_hkv8_len4096_page16")


def varlen_causal_gqa(seed=6):
    """Packed batch of 16 causal GQA sequences (Hq=32, Hkv=8), self attention
    with lengths iid U{1..8192}: a stand-in for a batch of prompts of mixed
    lengths without padding."""
    lens = _rng(seed, _S_VLENS).integers(1, 8193, size=16)
    return varlen_inputs(lens, lens, 32, 8, causal=True, seed=seed,
                         name="varlen_causal_gqa_b16_hq32_hkv8_len8192")


def headdim64_causal_gqa(seed=7):
    """Causal GQA prefill with head dim 64: B=8, Hq=32, Hkv=8, S=8192, BSHD
    (the causal GQA workload's shape at the smaller head size)."""
    return prefill_inputs(8, 32, 8, 8192, 8192, layout=BSHD, causal=True, seed=seed, d=64,
                          name="gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd")


def e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as OCP E4M3 (FN) bytes, round to nearest even,
    with torch's float8_e4m3fn conversion; values beyond +-448 are clipped to
    +-448 first (the conversion would give the NaN encoding)."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


@dataclass
class Fp8Prefill:
    """One FP8 prefill problem: q/k/v are E4M3 byte arrays in `layout`, each
    with a float32 descale factor (real value = descale * decoded byte)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    layout: int
    causal: bool
    scale: float
    descale_q: float
    descale_k: float
    descale_v: float
    name: str = ""

    @property
    def flops(self) -> float:
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * D
        return f / 2 if self.causal else f


def fp8_prefill_inputs(B, Hq, Hkv, Sq, Sk, *, layout=BSHD, causal=False, seed=0, scale=None,
                       descales=(1.0, 1.0, 1.0), amp=(1.0, 1.0, 1.0), name="") -> Fp8Prefill:
    """Draw Q, K, V iid N(0, 1) times amp (per tensor) in float32 and encode
    them as E4M3; `descales` are stored beside them as float32.  A small amp
    puts many values among the E4M3 subnormals (|x| < 2^-6)."""
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = e4m3_bytes(amp[0] * _normal(seed, _S_F8Q, layout_shape(layout, B, Hq, Sq)))
    k = e4m3_bytes(amp[1] * _normal(seed, _S_F8K, layout_shape(layout, B, Hkv, Sk)))
    v = e4m3_bytes(amp[2] * _normal(seed, _S_F8V, layout_shape(layout, B, Hkv, Sk)))
    dq, dk, dv = (float(np.float32(x)) for x in descales)
    return Fp8Prefill(q, k, v, B, Hq, Hkv, Sq, Sk, layout, bool(causal), float(scale), dq, dk, dv,
                      name=name)


def fp8_mha_prefill(seed=8):
    """The MHA prefill workload's shape (B=4, H=32, S=4096, BHSD, non-causal)
    with E4M3 inputs drawn from N(0, 1) and descales 1."""
    return fp8_prefill_inputs(4, 32, 32, 4096, 4096, layout=BHSD, seed=seed,
                              name="fp8_mha_prefill_b4_h32_s4096_bhsd")


def fp8_causal_gqa(seed=9):
    """The causal GQA workload's shape (B=8, Hq=32, Hkv=8, S=8192, BSHD) with
    E4M3 inputs drawn from N(0, 1) and descales 1."""
    return fp8_prefill_inputs(8, 32, 8, 8192, 8192, layout=BSHD, causal=True, seed=seed,
                              name="fp8_gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd")
