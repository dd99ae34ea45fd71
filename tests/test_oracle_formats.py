"""Pins of the oracle's number formats and dequant rule against what the pages
and the formats' definitions fix: a library E4M3 decoder, the E2M1 table of the
OCP MX specification, the divisor 2688 printed on the pack page, and exact
rational rounding."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact


def test_e4m3_matches_library_decoder():
    lib = exact.e4m3_table()
    for b in range(256):
        v = oracle.e4m3_value(b)
        if b in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(lib[b])
        else:
            assert v == lib[b], hex(b)
            assert math.copysign(1.0, v) == math.copysign(1.0, lib[b])


def test_e2m1_matches_ocp_table():
    tab = exact.e2m1_table()
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == tab[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, tab[c])


def test_divisor_is_max_e4m3_times_max_e2m1():
    # The pack page's global-scales bullet divides g by 2688; that is the product
    # of the largest E4M3FN magnitude and the largest E2M1 magnitude, which pins
    # both variants (E4M3FNUZ would give 240 * 6, E5M2 57344 * 6).
    nums = json.load(open(os.path.join(exact.GOLDEN_DIR, "pack_numbers.json")))
    finite = [abs(oracle.e4m3_value(b)) for b in range(256) if b not in (0x7F, 0xFF)]
    assert max(finite) * max(abs(oracle.e2m1_value(c)) for c in range(16)) == nums["global_divisor"]["value"]


def test_unit_products_exact_in_bf16():
    # every E2M1 x E4M3 product has at most 6 significant bits, so it is exact
    # in bf16 (8 bits): the bf16 "unit" value loses nothing
    for c in range(16):
        for b in range(256):
            if b in (0x7F, 0xFF):
                continue
            q = Fraction(oracle.e2m1_value(c)) * Fraction(oracle.e4m3_value(b))
            bits = exact.round_bf16_bits(q)
            assert Fraction(exact.bf16_value(bits)) == q


def _g_samples():
    rng = np.random.default_rng(7)
    g = list((2688.0 * rng.uniform(0.5, 2.0, 300)).astype(np.float32))
    g += [np.float32(2688.0), np.float32(1.0), np.float32(3e-38), np.float32(1e30),
          np.float32(1344.0), np.float32(5376.0), np.nextafter(np.float32(2688.0), np.float32(0))]
    return g


def test_global_factor_is_correctly_rounded_division():
    for g in _g_samples():
        t = np.float32(oracle.global_factor(float(g)))
        assert t == exact.round_f32(Fraction(float(g)) / 2688), g


def test_block_scale_and_weight_single_roundings():
    rng = np.random.default_rng(11)
    gs = _g_samples()[:40]
    for g in gs:
        t = Fraction(float(exact.round_f32(Fraction(float(g)) / 2688)))
        for b in list(rng.integers(0, 0x7F, 12)) + [0x01, 0x08, 0x38, 0x7E, 0x81, 0xFE]:
            S = np.float32(oracle.block_scale(int(b), float(g)))
            want_S = exact.round_f32(Fraction(oracle.e4m3_value(int(b))) * t)
            assert S == want_S
            for c in range(16):
                w = np.float32(oracle.weight(c, int(b), float(g)))
                assert w == exact.round_f32(Fraction(oracle.e2m1_value(c)) * Fraction(float(want_S)))


def test_unit_scale_and_g_2688_give_e2m1_exactly():
    # e4m3 byte 0x38 is 1.0 and g = 2688 makes t = 1: w is the E2M1 value itself
    tab = exact.e2m1_table()
    for c in range(16):
        assert oracle.weight(c, 0x38, 2688.0) == tab[c]


def test_bf16_rounding_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # include exact ties of the bf16 grid and values near the overflow edge
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.array([3.3895314e38, -3.3895314e38, 1e-40, -1e-45], np.float32)])
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_of_f64_values_is_single_rounding():
    # values between two f32 neighbours where f64 -> f32 -> bf16 would round twice
    rng = np.random.default_rng(5)
    for _ in range(300):
        base = float(np.float32(rng.normal()))
        v = base + rng.normal() * abs(base) * 2.0**-12
        assert int(oracle.f64_to_bf16([v])[0]) == exact.round_bf16_bits(Fraction(v))
    # an exact tie in f64 that is not a tie after rounding to f32 first
    v = 1.0 + 2.0**-8 + 2.0**-40
    assert int(oracle.f64_to_bf16([v])[0]) == exact.round_bf16_bits(Fraction(v))
