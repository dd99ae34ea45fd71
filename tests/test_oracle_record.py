"""Pins of the oracle's record layout against the numbers the pack page prints,
and of nibble order / orientation by constructed one-hot records."""
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle
from tests import exact

NUMS = json.load(open(os.path.join(exact.GOLDEN_DIR, "pack_numbers.json")))


def test_record_bytes_and_stride_match_pack_page():
    H, I = NUMS["hidden"]["value"], NUMS["intermediate"]["value"]
    off, nbytes, stride = oracle.record_layout(H, I)
    assert nbytes == NUMS["record_bytes"]["value"]
    assert stride == NUMS["record_stride"]["value"]
    assert stride % 4096 == 0 and stride - nbytes < 4096


def test_bank_and_row_sizes_match_pack_page():
    H, I = NUMS["hidden"]["value"], NUMS["intermediate"]["value"]
    _, nbytes, stride = oracle.record_layout(H, I)
    assert NUMS["records"]["value"] == 49 * 256
    assert round(NUMS["records"]["value"] * stride / 1e9, 1) == NUMS["experts_bin_GB"]["value"]
    assert 49 * stride == NUMS["row_bytes"]["value"]
    # the seed load counts record bytes, not strides: 198.34 GB (strides: 198.37)
    assert round(NUMS["seed_records"]["value"] * nbytes / 1e9, 1) == NUMS["seed_records"]["GB"]
    assert round(NUMS["seed_records"]["value"] * stride / 1e9, 1) != NUMS["seed_records"]["GB"]


def test_mid_bytes_match_vq_page():
    I = NUMS["intermediate"]["value"]
    assert 8 * I * 2 == NUMS["mid_bytes_8_experts"]["value"]


def test_tiny_layout_and_alignment():
    off, nbytes, stride = oracle.record_layout(256, 128)
    assert nbytes == 55308 and stride == 57344
    off, nbytes, stride = oracle.record_layout(5120, 2560)
    # code and scale parts start on 4 KiB boundaries; the globals close the record
    assert all(o % 4096 == 0 for o in off[:6])
    assert off[6:] == [nbytes - 12, nbytes - 8, nbytes - 4]


def test_bad_shapes_rejected():
    for H, I in [(0, 16), (16, 0), (24, 16), (16, 8)]:
        try:
            oracle.record_layout(H, I)
        except ValueError:
            continue
        raise AssertionError((H, I))


def _zero_parts(H, I):
    codes = [np.zeros((I, H // 8), np.uint32), np.zeros((I, H // 8), np.uint32), np.zeros((H, I // 8), np.uint32)]
    scales = [np.full((I, H // 16), 0x38, np.uint8), np.full((I, H // 16), 0x38, np.uint8),
              np.full((H, I // 16), 0x38, np.uint8)]
    return codes, scales


def test_one_hot_code_lands_at_its_row_and_column():
    # Reading: element 8q + j of a row is nibble j (bits 4j..4j+3) of word q,
    # rows are outputs, columns inputs. With unit scales and g = 2688 a single
    # code 7 (= 6.0) must appear at exactly one (row, column).
    H, I = 64, 32
    for p, (r, c) in [(0, (5, 13)), (1, (31, 63)), (2, (40, 9)), (0, (0, 0))]:
        codes, scales = _zero_parts(H, I)
        codes[p][r, c // 8] = np.uint32(7 << (4 * (c % 8)))
        rec = oracle.pack_record(H, I, codes, scales, [2688.0, 2688.0, 2688.0])
        for q in range(3):
            w, u = oracle.dequant_projection(rec, H, I, q)
            nz = np.argwhere(w != 0)
            if q == p:
                assert nz.tolist() == [[r, c]] and w[r, c] == 6.0
                assert u[r, c] == 0x40C0  # bf16 6.0
            else:
                assert nz.size == 0


def test_block_scale_covers_sixteen_inputs():
    H, I = 64, 32
    codes, scales = _zero_parts(H, I)
    codes[0][:] = np.uint32(0x22222222)  # every gate weight code 2 (= 1.0)
    scales[0][3, 2] = 0x40  # e4m3 2.0 on row 3, inputs 32..47
    rec = oracle.pack_record(H, I, codes, scales, [2688.0, 2688.0, 2688.0])
    w, _ = oracle.dequant_projection(rec, H, I, 0)
    want = np.ones((I, H), np.float32)
    want[3, 32:48] = 2.0
    assert np.array_equal(w, want)


def test_pack_bytes_layout():
    H, I = 32, 16
    rng = np.random.default_rng(0)
    codes = [rng.integers(0, 2**32, s, dtype=np.uint64).astype(np.uint32) for s in [(I, H // 8), (I, H // 8), (H, I // 8)]]
    scales = [rng.integers(0, 0x7F, s).astype(np.uint8) for s in [(I, H // 16), (I, H // 16), (H, I // 16)]]
    g = np.array([1000.0, 2000.0, 3000.0], np.float32)
    rec = oracle.pack_record(H, I, codes, scales, g)
    off, nbytes, stride = oracle.record_layout(H, I)
    assert rec.size == stride and not rec[nbytes:].any()
    for p in range(3):
        assert rec[off[2 * p]:off[2 * p] + codes[p].nbytes].tobytes() == codes[p].astype("<u4").tobytes()
        assert rec[off[2 * p + 1]:off[2 * p + 1] + scales[p].nbytes].tobytes() == scales[p].tobytes()
        assert rec[off[6 + p]:off[6 + p] + 4].view("<f4")[0] == g[p]


def _unit_want(codes_row_words, scale_row, in_):
    """bf16 bits of e2m1(c) * e4m3(s) for one row, from the OCP E2M1 table, a
    library E4M3 decoder and exact rational rounding (no oracle code)"""
    e2m1 = exact.e2m1_table()
    e4m3 = exact.e4m3_table()
    out = np.empty(in_, np.uint16)
    for c in range(in_):
        code = (int(codes_row_words[c // 8]) >> (4 * (c % 8))) & 15
        a, b = e2m1[code], float(e4m3[int(scale_row[c // 16])])
        q = Fraction(a) * Fraction(b)
        # a zero product takes the sign rule of IEEE multiplication
        neg = (math.copysign(1.0, a) < 0) != (math.copysign(1.0, b) < 0)
        out[c] = exact.round_bf16_bits(q) if q != 0 else (0x8000 if neg else 0)
    return out


def test_unit_values_follow_codes_and_scales_not_g():
    # The bf16 unit value of a weight is e2m1(code) * e4m3(block scale), exact
    # ([PACK] "What this pack holds", global-scales bullet: the global factor
    # g / 2688 multiplies e4m3(scale) on top of it). Random codes, every finite
    # E4M3 scale byte of either sign (subnormals 0x01..0x07 included) and
    # several g far from 2688: every element is compared, and the same codes
    # and scales under another g give the same unit values.
    H, I = 64, 48
    rng = np.random.default_rng(2024)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    codes = [rng.integers(0, 2**32, s, dtype=np.uint64).astype(np.uint32) for s in [(I, H // 8), (I, H // 8), (H, I // 8)]]
    scales = [rng.choice(finite, s) for s in [(I, H // 16), (I, H // 16), (H, I // 16)]]
    scales[0].flat[:254] = finite  # every finite byte at least once
    scales[2].flat[:8] = np.arange(8, dtype=np.uint8)  # zero and the subnormals
    units = []
    for g in ([1000.5, 2688.0 * 1.75, 37.0], [5000.0, 0.03125, 2688.0 * 0.6]):
        rec = oracle.pack_record(H, I, codes, scales, np.array(g, np.float32))
        units.append([oracle.dequant_projection(rec, H, I, p)[1] for p in range(3)])
    for p in range(3):
        out, in_ = oracle.proj_shape(H, I, p)
        for r in range(out):
            want = _unit_want(codes[p][r], scales[p][r], in_)
            assert np.array_equal(units[0][p][r], want), (p, r)
        assert np.array_equal(units[0][p], units[1][p]), p
