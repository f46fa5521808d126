"""The oracle's bf16 rounding rules against their pins (CPU only), and planted
mistakes in a private copy of the rounding module that the pins must catch."""
import importlib.util
import os
import types

import numpy as np
import pytest

import oracle.rounding as rnd
import rounding_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "rounding.py")


@pytest.mark.parametrize("pin", rounding_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(rnd)


def test_unknown_mode_and_unrepresentable_values_raise():
    with pytest.raises(ValueError):
        rnd.round_bf16(np.array([1.0]), "rtp")
    with pytest.raises(ValueError):
        rnd.bf16_bits(np.array([1.0 + 2.0 ** -9]))


def test_nan_stays_nan():
    for m in rnd.MODES:
        assert np.isnan(rnd.round_bf16(np.array([np.nan]), m)[0])
    assert rnd.bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def mutant(old: str, new: str) -> types.ModuleType:
    src = open(SRC).read()
    assert old in src, old
    m = types.ModuleType("rounding_mutant")
    exec(compile(src.replace(old, new, 1), "rounding_mutant", "exec"), m.__dict__)
    return m


MUTANTS = {
    "rtne_ties_up": ("((frac > 0.5) | ((frac == 0.5) & odd))", "(frac >= 0.5)"),
    "rtne_ties_down": ("((frac > 0.5) | ((frac == 0.5) & odd))", "(frac > 0.5)"),
    "rtna_ties_toward_plus_inf": ("r = n + (frac >= 0.5)",
                                  "r = n + ((frac > 0.5) | ((frac == 0.5) & (x[fin] > 0)))"),
    "rtz_toward_minus_inf": ("        r = n\n", "        r = n + (x[fin] < 0)\n"),
    "no_subnormal_spacing": ("np.maximum(e2.astype(np.int64) - 1, -126)",
                             "e2.astype(np.int64) - 1"),
    "spacing_off_by_one": ("(e - 7)", "(e - 8)"),
    "nearest_saturates": ("np.where(mag > BF16_MAX, np.inf, mag)", "np.minimum(mag, BF16_MAX)"),
    "rtz_overflows": ("mag = np.minimum(mag, BF16_MAX)", "mag = mag"),
    "sign_dropped_on_zero": ("np.copysign(mag, x[fin])",
                             "np.where(mag == 0, 0.0, np.copysign(mag, x[fin]))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    m = mutant(*MUTANTS[name])
    caught = []
    for pin in rounding_pins.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError):   # a wrong value, or a non-bf16 result
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
