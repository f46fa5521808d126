"""Pins of the bf16 rounding rules of the oracle (oracle.rounding), as
functions of the module under test so that planted mistakes can be run
through the same checks.  Each pin fixes the rules by something other than the
oracle's own arithmetic: hand-derived worked cases, an independent library
conversion (torch's float32 -> bfloat16 is round-to-nearest-even), the bit
definition of truncation, and properties every correct rounding has."""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "bf16_rounding_cases.txt")


def worked_cases():
    xs, exp = [], []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        xs.append(float.fromhex(f[0]) if "inf" not in f[0] else float(f[0]))
        exp.append([int(t, 16) for t in f[1:4]])
    return np.array(xs), np.array(exp, dtype=np.uint16)


def _f32_samples(seed: int, n: int = 200_000) -> np.ndarray:
    """float32 values over every binade: random bit patterns (finite), exact
    ties and quarter points of bf16 spacings, subnormals and near-overflow."""
    r = np.random.default_rng(seed)
    bits = r.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]
    hi = bits & 0xFFFF0000
    extra = np.concatenate([hi | 0x8000, hi | 0x4000, hi | 0xC000, hi | 0x7FFF, hi | 0x8001])
    extra = extra[(extra & 0x7F800000) != 0x7F800000]
    sub = r.integers(0, 2 ** 23, size=2000, dtype=np.uint64).astype(np.uint32)
    top = (0x7F7F0000 + r.integers(0, 2 ** 16, size=2000, dtype=np.uint64)).astype(np.uint32)
    allb = np.concatenate([bits, extra, sub, sub | 0x80000000, top, top | 0x80000000])
    return allb.view(np.float32).astype(np.float64)


def pin_worked_cases(rnd):
    xs, exp = worked_cases()
    for col, mode in enumerate(("rtne", "rtna", "rtz")):
        got = rnd.bf16_bits(rnd.round_bf16(xs, mode))
        bad = np.nonzero(got != exp[:, col])[0]
        assert bad.size == 0, (mode, [(xs[i].hex(), hex(got[i]), hex(exp[i, col])) for i in bad])


def pin_rtne_is_torch_conversion(rnd):
    x = _f32_samples(1)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    ref = ref.numpy().view(np.uint16)
    got = rnd.bf16_bits(rnd.round_bf16(x, "rtne"))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(x[i].hex(), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def pin_rtz_is_bit_truncation(rnd):
    """For float32 inputs, dropping the low 16 bits of the sign-magnitude
    encoding is truncation toward zero."""
    x = _f32_samples(2)
    ref = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = rnd.bf16_bits(rnd.round_bf16(x, "rtz"))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(x[i].hex(), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def _next_up(v: np.ndarray) -> np.ndarray:
    """The bf16 value after v >= 0 (by the bit pattern; max finite -> inf)."""
    b = v.astype(np.float32).view(np.uint32) >> 16
    return ((b + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def pin_properties(rnd):
    """On float64 values (not only float32 ones): every result is a bf16
    value; RTZ never grows the magnitude and the next bf16 value is above |x|;
    the nearest rules stay within half a spacing of x and agree except on
    exact ties, where RTNE's last bit is 0 and RTNA's magnitude is the larger;
    all three are odd functions and monotone."""
    r = np.random.default_rng(3)
    x = np.ldexp(r.uniform(0.5, 1.0, 100_000), r.integers(-140, 129, 100_000))
    x *= r.choice([-1.0, 1.0], x.size)
    # exact ties: k + 1/2 spacings in binade 2^e, and in the subnormal range
    ties = np.ldexp(r.integers(128, 256, 5000) + 0.5, r.integers(-126, 127, 5000) - 7)
    sub_ties = np.ldexp(r.integers(0, 128, 1000) + 0.5, -133)
    x = np.concatenate([x, ties, -ties, sub_ties, -sub_ties])
    a = np.abs(x)
    fin = a <= rnd.BF16_MAX
    res = {m: rnd.round_bf16(x, m) for m in ("rtne", "rtna", "rtz")}
    for m, v in res.items():
        rnd.bf16_bits(v[np.isfinite(v)])                      # representable
        assert np.array_equal(rnd.round_bf16(-x, m), -v), m   # odd
        vs = v[np.argsort(x, kind="stable")]
        assert np.all(vs[1:] >= vs[:-1]), m                    # monotone
    z = np.abs(res["rtz"])
    assert np.all(z <= a)
    assert np.all(_next_up(z)[fin] > a[fin])
    half = rnd.spacing(a) / 2
    for m in ("rtne", "rtna"):
        assert np.all(np.abs(res[m] - x)[fin] <= half[fin]), m
    tie = np.abs(np.abs(res["rtz"] - x) - half) == 0
    tie &= fin
    same = res["rtne"] == res["rtna"]
    assert np.all(same[~tie])
    ne = np.abs(res["rtne"][tie]).astype(np.float32).view(np.uint32)
    assert np.all(((ne >> 16) & 1) == 0)
    assert np.all(np.abs(res["rtna"][tie]) > a[tie])
    assert tie.sum() >= 10_000


ALL_PINS = [pin_worked_cases, pin_rtne_is_torch_conversion, pin_rtz_is_bit_truncation,
            pin_properties]
