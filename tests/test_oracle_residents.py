"""Pins of the oracle's q8 quantizer (the pack page's q8 rule), its affine8_g64
linear and the weightless RMS norm: exact invariants, constructed ties,
numbers printed on the pack page, and float64 numpy references."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact

NUMS = json.load(open(os.path.join(exact.GOLDEN_DIR, "pack_numbers.json")))


def _codes_u8(codes, N, K):
    return codes.view(np.uint8).reshape(N, K)  # little-endian: first code in the low byte


def _check_group(vals_bits, q, sbits, bbits):
    v = [Fraction(exact.bf16_value(b)) for b in vals_bits]
    mn, mx = min(v), max(v)
    s, b = Fraction(exact.bf16_value(sbits)), Fraction(exact.bf16_value(bbits))
    assert b == mn  # bias is the group minimum, exactly
    d = mx - mn
    if d == 0:
        assert s == 0 and all(int(c) == 0 for c in q)
        return
    assert 255 * s >= d  # no value clipped
    prev = Fraction(exact.bf16_value(int(sbits) - 1))
    assert 255 * prev < d  # the scale is the smallest such bf16
    for val, c in zip(v, q):
        c = int(c)
        assert 0 <= c <= 255
        err = abs(val - (b + c * s))
        assert 2 * err <= s  # within half a scale
        if 2 * err == s:  # an exact tie: the even step
            assert c % 2 == 0


def test_q8_invariants_on_synthetic_weights():
    N, K = 24, 512
    v = synth.resident_weights(3, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    q = _codes_u8(codes, N, K)
    for n in range(N):
        for g in range(K // 64):
            _check_group(v[n, 64 * g:64 * g + 64], q[n, 64 * g:64 * g + 64], scales[n, g], biases[n, g])


def test_q8_adversarial_groups():
    rng = np.random.default_rng(8)
    groups = []
    groups.append(np.full(64, 0x3F80, np.uint16))  # constant group
    groups.append(np.zeros(64, np.uint16))  # all +0
    g = rng.integers(0, 0x7F00, 64).astype(np.uint16)  # wide positive range
    groups.append(g)
    g = (rng.integers(0, 0x7F00, 64).astype(np.uint16) | 0x8000)  # negative values
    groups.append(g)
    g = synth.to_bf16_bits(rng.normal(size=64) * 1e-38)  # subnormal-scale range
    groups.append(g)
    # constructed exact ties: min 0, max 255 * 2^-7 so the scale is 2^-7,
    # values (n + 1/2) * 2^-7 must round to the even step
    s = 2.0**-7
    vals = [0.0, 255 * s] + [(n + 0.5) * s for n in range(1, 63)]
    tie = synth.to_bf16_bits(np.array(vals))
    assert np.array_equal(oracle.bf16_to_f32(tie).astype(np.float64), np.array(vals))
    groups.append(tie)
    v = np.stack(groups)
    codes, scales, biases = oracle.q8_quantize(v)
    q = _codes_u8(codes, v.shape[0], 64)
    for i in range(v.shape[0]):
        _check_group(v[i], q[i], scales[i, 0], biases[i, 0])
    assert exact.bf16_value(scales[-1, 0]) == s
    assert [int(c) for c in q[-1, 2:]] == [n + (n % 2) for n in range(1, 63)]


def test_q8_bytes_per_weight_match_pack_page():
    # 8-bit codes plus a bf16 scale and bias per 64 weights against 2 bytes of
    # bf16: (1 + 4/64) / 2 = 0.53125, the pack page's 7.62 GB / 14.35 GB
    N, K = 64, 128
    codes, scales, biases = oracle.q8_quantize(synth.resident_weights(1, N, K))
    ratio = (codes.nbytes + scales.nbytes + biases.nbytes) / (N * K * 2)
    q = NUMS["q8_resident_GB"]
    assert ratio == 0.53125
    assert abs(ratio - q["value"] / q["bf16_GB"]) < 0.005 / q["bf16_GB"] + 0.005 / q["value"]


def test_q8_relative_rms_error_is_small():
    # context only: the pack page reports 0.54-0.63 % on Beam's weights; on
    # N(0, 0.02) groups of 64 the rounding error is about scale / sqrt(12)
    N, K = 64, 1024
    v = synth.resident_weights(2, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    q = _codes_u8(codes, N, K).astype(np.float64)
    s = np.repeat(oracle.bf16_to_f32(scales).astype(np.float64), 64, axis=1)
    b = np.repeat(oracle.bf16_to_f32(biases).astype(np.float64), 64, axis=1)
    vf = oracle.bf16_to_f32(v).astype(np.float64)
    rel = np.sqrt(np.mean((s * q + b - vf) ** 2) / np.mean(vf**2))
    assert 0.001 < rel < 0.01, rel


def test_affine8_linear_matches_numpy_dense():
    T, K, N = 3, 256, 96
    v = synth.resident_weights(4, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(4, T, K)
    yf, yb = oracle.affine8_linear(x, codes, scales, biases)
    q = _codes_u8(codes, N, K).astype(np.float64)
    W = q * np.repeat(oracle.bf16_to_f32(scales).astype(np.float64), 64, axis=1) + \
        np.repeat(oracle.bf16_to_f32(biases).astype(np.float64), 64, axis=1)
    ref = oracle.bf16_to_f32(x).astype(np.float64) @ W.T
    assert np.all(np.abs(yf - ref.astype(np.float32)) <= np.spacing(np.abs(ref.astype(np.float32))))
    # one-hot input selects a dequantized weight column exactly
    x1 = np.zeros((1, K), np.uint16)
    x1[0, 77] = 0x3F80
    y1, _ = oracle.affine8_linear(x1, codes, scales, biases)
    assert np.array_equal(y1[0], W[:, 77].astype(np.float32))
    with pytest.raises(ValueError):
        oracle.affine8_linear(x[:, :100], codes[:, :25], scales, biases)


def test_rmsnorm_matches_numpy():
    x = synth.activations(9, 4, 512)
    y = oracle.rmsnorm(x, 1e-6)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    ref = xf / np.sqrt(np.mean(xf**2, axis=1, keepdims=True) + 1e-6)
    got = oracle.bf16_to_f32(y).astype(np.float64)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + 1e-30)
