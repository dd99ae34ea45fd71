"""Pins of the oracle's MoE layer: an exact-rational brute force on tiny layers,
a numpy float64 dense reference with independent decoders, and the special
cases that reduce the layer to something known."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from tests import exact

E2M1 = exact.e2m1_table()
E4M3 = exact.e4m3_table()


def make_records(seed, E, H, I):
    recs, parts = {}, {}
    for e in range(E):
        codes, scales, g = synth.expert_parts(seed, e, H, I)
        c = [x.numpy().view(np.uint32) for x in codes]
        s = [x.numpy() for x in scales]
        recs[e] = oracle.pack_record(H, I, c, s, g)
        parts[e] = (c, s, g)
    return recs, parts


def dense_weights_np(codes, scales, g):
    """Independent decode: nibbles by numpy shifts on the U32 words, E2M1 from the
    golden table, E4M3 from torch's float8 dtype, f32 products by numpy."""
    rows, wpr = codes.shape
    nib = np.stack([(codes >> np.uint32(4 * j)) & np.uint32(15) for j in range(8)], axis=-1).reshape(rows, wpr * 8)
    e2 = np.array(E2M1, np.float32)[nib]
    sc = E4M3[scales].astype(np.float32)
    t = np.float32(g) / np.float32(2688.0)
    S = (sc * t).astype(np.float32)
    return (e2 * np.repeat(S, 16, axis=1)).astype(np.float32)


def test_exact_brute_force_tiny_layer():
    H, I, E, k, T = 32, 16, 4, 2, 2
    recs, parts = make_records(21, E, H, I)
    x = synth.activations(21, T, H)
    lg = np.random.default_rng(2).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    yf, yb, mid = oracle.moe_forward(recs, E, H, I, x, idx, w, want_mid=True)
    xv = [[Fraction(exact.bf16_value(b)) for b in row] for row in x]

    def W(e, p):
        c, s, g = parts[e]
        t = Fraction(float(exact.round_f32(Fraction(float(g[p])) / 2688)))
        rows, wpr = c[p].shape
        M = []
        for r in range(rows):
            row = []
            for col in range(wpr * 8):
                code = (int(c[p][r, col // 8]) >> (4 * (col % 8))) & 15
                S = Fraction(float(exact.round_f32(Fraction(float(E4M3[s[p][r, col // 16]])) * t)))
                row.append(Fraction(float(exact.round_f32(Fraction(E2M1[code]) * S))))
            M.append(row)
        return M

    Ws = {e: [W(e, p) for p in range(3)] for e in set(idx.ravel().tolist())}
    for t in range(T):
        acc = Fraction(0)
        for j in range(k):
            e = int(idx[t, j])
            Wg, Wu, Wd = Ws[e]
            gate = [float(exact.round_f32(sum(a * b for a, b in zip(row, xv[t])))) for row in Wg]
            up = [float(exact.round_f32(sum(a * b for a, b in zip(row, xv[t])))) for row in Wu]
            mids = []
            for i in range(I):
                sv = gate[i] * scipy.special.expit(gate[i]) * up[i]
                mb = exact.round_bf16_bits(Fraction(sv))
                assert exact.bf16_value(mb) == exact.bf16_value(mid[t * k + j, i])
                mids.append(Fraction(exact.bf16_value(mb)))
            d = [sum(a * b for a, b in zip(row, mids)) for row in Wd]
            if j == 0:
                acc = [Fraction(float(w[t, j])) * v for v in d]
            else:
                acc = [a + Fraction(float(w[t, j])) * v for a, v in zip(acc, d)]
        for h in range(H):
            want = exact.round_f32(acc[h])
            assert abs(float(yf[t, h]) - float(want)) <= float(np.spacing(np.abs(want))), (t, h)
            assert abs(int(yb[t, h]) - exact.round_bf16_bits(acc[h])) <= 1


def _numpy_layer(parts, x, idx, w, H, I, residual=None):
    T, k = idx.shape
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    y = np.zeros((T, H)) if residual is None else oracle.bf16_to_f32(residual).astype(np.float64)
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e not in cache:
                c, s, g = parts[e]
                cache[e] = [dense_weights_np(c[p], s[p], g[p]).astype(np.float64) for p in range(3)]
            Wg, Wu, Wd = cache[e]
            gate = (Wg @ xf[t]).astype(np.float32).astype(np.float64)
            up = (Wu @ xf[t]).astype(np.float32).astype(np.float64)
            sw = gate * scipy.special.expit(gate) * up
            mid = torch.from_numpy(sw).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
            y[t] += float(w[t, j]) * (Wd @ mid)
    return y


def test_tiny_config_matches_numpy_dense_reference():
    # the tiny layer config: H=256, I=128, E=16, top-2, T=4
    H, I, E, k, T = 256, 128, 16, 2, 4
    recs, parts = make_records(0, E, H, I)
    x = synth.activations(0, T, H)
    Wr = synth.router_weights(0, H, E)
    idx, w = oracle.route_topk(oracle.router_logits(x, Wr), k)
    yf, yb = oracle.moe_forward(recs, E, H, I, x, idx, w)
    ref = _numpy_layer(parts, x, idx, w, H, I)
    # the reference rounds mids f64 -> f32 -> bf16 (a rare double rounding) and
    # sums in another order; bound the difference far below the layer tolerance
    rel = np.linalg.norm(yf - ref) / np.linalg.norm(ref)
    assert rel < 1e-5, rel


def test_unit_scales_one_hot_input_and_single_expert():
    # All scales 1.0 and g = 2688 make W the E2M1 values; a one-hot input picks
    # one weight column; k = 1 makes the routing weight exactly 1. Then
    # mid_i = bf16(silu(Wg[i,h]) * Wu[i,h]) and y = Wd @ mid exactly.
    H, I, E = 64, 32, 3
    rng = np.random.default_rng(4)
    recs, dense = {}, {}
    for e in range(E):
        codes = [rng.integers(0, 2**32, s, dtype=np.uint64).astype(np.uint32) for s in [(I, H // 8), (I, H // 8), (H, I // 8)]]
        scales = [np.full(s, 0x38, np.uint8) for s in [(I, H // 16), (I, H // 16), (H, I // 16)]]
        recs[e] = oracle.pack_record(H, I, codes, scales, [2688.0] * 3)
        dense[e] = [oracle.dequant_projection(recs[e], H, I, p, want_unit=False)[0] for p in range(3)]
        for p in range(3):
            assert set(np.unique(dense[e][p]).tolist()) <= set(E2M1)
    h = 17
    x = np.zeros((1, H), np.uint16)
    x[0, h] = 0x3F80  # bf16 1.0
    for e in range(E):
        idx = np.array([[e]], np.int32)
        wgt = np.array([[1.0]], np.float32)
        yf, yb, mid = oracle.moe_forward(recs, E, H, I, x, idx, wgt, want_mid=True)
        Wg, Wu, Wd = dense[e]
        sw = [float(Wg[i, h]) * scipy.special.expit(float(Wg[i, h])) * float(Wu[i, h]) for i in range(I)]
        want_mid = [exact.round_bf16_bits(Fraction(v)) for v in sw]
        # compare values: the oracle keeps IEEE signed zeros, Fractions have none
        assert [exact.bf16_value(b) for b in mid[0]] == [exact.bf16_value(b) for b in want_mid]
        mv = [Fraction(exact.bf16_value(b)) for b in want_mid]
        for r in range(H):
            acc = sum(Fraction(float(Wd[r, i])) * mv[i] for i in range(I))
            assert yf[0, r] == exact.round_f32(acc)


def test_residual_and_accumulation_modes():
    H, I, E, k, T = 128, 64, 8, 2, 3
    recs, _ = make_records(5, E, H, I)
    x = synth.activations(5, T, H)
    r = synth.activations(6, T, H)
    lg = np.random.default_rng(1).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    y0, _ = oracle.moe_forward(recs, E, H, I, x, idx, w)
    y1, _ = oracle.moe_forward(recs, E, H, I, x, idx, w, residual=r)
    assert np.allclose(y1 - y0, oracle.bf16_to_f32(r), rtol=0, atol=1e-4 * np.abs(y0).max())
    y32, _ = oracle.moe_forward(recs, E, H, I, x, idx, w, acc=oracle.ACC_F32)
    rel = np.linalg.norm(y32 - y0) / np.linalg.norm(y0)
    assert rel < 1e-4, rel


def test_bad_arguments_rejected():
    H, I, E = 32, 16, 2
    recs, _ = make_records(1, E, H, I)
    x = synth.activations(1, 1, H)
    with pytest.raises(ValueError):
        oracle.moe_forward(recs, E, H, I, x, np.array([[2]], np.int32), np.ones((1, 1), np.float32))
    with pytest.raises(ValueError):
        oracle.moe_forward({0: recs[0]}, E, H, I, x, np.array([[1]], np.int32), np.ones((1, 1), np.float32))
