"""Pins of the oracle's 8-dim VQ expert format ("Beam-1.0-501B-A23B VQ GGUF",
"Recipe", routed-experts bullet): the F16 gain and E4M3 codeword decoders, the
12-bit index stream, the record and codebook sizes against the page's numbers,
the exact weight rule, and the layer against a numpy dense reference."""
import json
import os
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import oracle
import synth
from tests import exact

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "vq_numbers.json")))


def test_f16_decoder_matches_numpy_on_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([oracle.f16_value(int(b)) for b in bits[fin]])
    assert np.array_equal(got, ref[fin])


def test_index_stream_against_python_bit_strings():
    rng = np.random.default_rng(1)
    for n_idx in (8, 16, 640, 320):
        row = rng.integers(0, 256, n_idx * 3 // 2, dtype=np.uint8)
        big = int.from_bytes(row.tobytes(), "little")
        for j in range(n_idx):
            assert oracle.vq_index(row, j) == (big >> (12 * j)) & 0xFFF


def test_sizes_match_the_page():
    assert GOLD["index_bits"]["value"] / GOLD["weights_per_index"]["value"] == GOLD["bits_per_weight"]["value"]
    # codebook: 2^12 codewords of 8 E4M3 bytes; the page's GB10 budget is the
    # mids plus the codebook plus the spare
    cb_bytes = (1 << GOLD["index_bits"]["value"]) * GOLD["weights_per_index"]["value"]
    assert cb_bytes == 32768
    assert GOLD["block_limit_bytes"]["value"] - GOLD["mid_bytes_8_experts"]["value"] - cb_bytes \
        == GOLD["spare_kib_12bit"]["value"] * 1024
    off, nbytes, stride = oracle.vq_layout(5120, 2560)
    idx_bytes = (off[1] - off[0]) + (off[3] - off[2]) + (off[5] - off[4])
    assert idx_bytes * 8 / (3 * 5120 * 2560) == GOLD["bits_per_weight"]["value"]
    assert nbytes == idx_bytes + 2 * (2560 + 2560 + 5120) and stride % 4096 == 0


def test_weight_rule_exact_and_one_hot():
    H, I = 128, 64
    cb = synth.vq_codebook(3)
    idx, gains = synth.vq_expert_parts(3, 0, H, I)
    rec = oracle.vq_pack_record(H, I, [a.numpy() for a in idx], gains)
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for p in range(3):
        W = oracle.vq_dequant_projection(rec, cb, H, I, p)
        rows, inn = W.shape
        rng = np.random.default_rng(p)
        for r, c in zip(rng.integers(0, rows, 50), rng.integers(0, inn, 50)):
            row = idx[p][r].numpy()
            j = int(c) // 8
            ci = (int.from_bytes(row.tobytes(), "little") >> (12 * j)) & 0xFFF
            want = Fraction(float(gains[p][r:r + 1].view(np.float16)[0])) * Fraction(float(e4[cb[ci, c % 8]]))
            assert Fraction(float(W[r, c])) == want
    # one-hot: gain 1.0, every index c -> the row repeats codeword c exactly
    z = [np.zeros((I, H * 3 // 16), np.uint8), np.zeros((I, H * 3 // 16), np.uint8), np.zeros((H, I * 3 // 16), np.uint8)]
    c = 2741
    for a in z:
        bits = 0
        for j in range(a.shape[1] * 2 // 3):
            bits |= c << (12 * j)
        a[:] = np.frombuffer(bits.to_bytes(a.shape[1], "little"), np.uint8)
    one = [np.full(a.shape[0], 0x3C00, np.uint16) for a in z]
    rec = oracle.vq_pack_record(H, I, z, one)
    W = oracle.vq_dequant_projection(rec, cb, H, I, 2)
    assert np.array_equal(W, np.tile(e4[cb[c]].astype(np.float32), (H, I // 8)))


def dense_vq_np(idx_bytes, gains, cb):
    """Independent decode: 12-bit fields from a Python big integer per row,
    E4M3 from torch's float8 dtype, F16 from numpy."""
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    rows, nb = idx_bytes.shape
    n_idx = nb * 2 // 3
    W = np.empty((rows, n_idx * 8), np.float32)
    for r in range(rows):
        big = int.from_bytes(idx_bytes[r].tobytes(), "little")
        ids = [(big >> (12 * j)) & 0xFFF for j in range(n_idx)]
        W[r] = (e4[cb[ids]].ravel() * float(gains[r:r + 1].view(np.float16)[0])).astype(np.float32)
    return W


def test_layer_against_numpy_dense_reference():
    H, I, E, k, T = 128, 64, 5, 2, 3
    cb = synth.vq_codebook(4)
    recs, dense = {}, {}
    for e in range(E):
        idx, gains = synth.vq_expert_parts(4, e, H, I)
        ib = [a.numpy() for a in idx]
        recs[e] = oracle.vq_pack_record(H, I, ib, gains)
        dense[e] = [dense_vq_np(ib[p], gains[p], cb) for p in range(3)]
    x = synth.activations(4, T, H)
    lg = np.random.default_rng(3).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    yf, yb = oracle.vq_moe_forward(recs, cb, E, H, I, x, idx, w)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            Wg, Wu, Wd = (m.astype(np.float64) for m in dense[int(idx[t, j])])
            g = (Wg @ xf[t]).astype(np.float32).astype(np.float64)
            u = (Wu @ xf[t]).astype(np.float32).astype(np.float64)
            mid = oracle.bf16_to_f32(oracle.f64_to_bf16(g * scipy.special.expit(g) * u)).astype(np.float64)
            acc += float(w[t, j]) * (Wd @ mid)
        np.testing.assert_allclose(yf[t], acc, rtol=1e-6, atol=1e-6 * np.abs(acc).max())
