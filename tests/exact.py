"""Exact-arithmetic helpers for the oracle pins (test-side, independent of the
oracle): rational values, correctly rounded to f32 or bf16 by comparing
candidate neighbours, and an E2M1 table read from the golden fixture."""
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN_DIR, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return [vals[c] for c in range(16)]


def e4m3_table():
    """E4M3FN decode by torch's float8_e4m3fn dtype (a library decoder)"""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _nearest(q: Fraction, cand_fn):
    """nearest representable value to q among the candidates, ties to even"""
    cands = cand_fn(q)
    best = None
    for c, even in cands:
        d = abs(Fraction(float(c)) - q)
        key = (d, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _f32_cands(q: Fraction):
    c = np.float32(float(q))
    out = []
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        bits = int(np.array(v, dtype=np.float32).view(np.uint32))
        out.append((np.float32(v), bits % 2 == 0))
    return out


def round_f32(q) -> np.float32:
    """f32 nearest to the rational q (ties to even)"""
    return _nearest(Fraction(q), _f32_cands)


def _bf16_from_bits(b):
    return np.array([b << 16], dtype=np.uint32).view(np.float32)[0]


def round_bf16_bits(q) -> int:
    """bf16 nearest to the rational q (ties to even), as bits"""
    q = Fraction(q)
    f = np.float32(float(q))
    b = int(np.array(f, dtype=np.float32).view(np.uint32)) >> 16
    best = None
    for cb in (b - 1, b, b + 1, b + 2):
        cb &= 0xFFFF
        v = _bf16_from_bits(cb)
        if not np.isfinite(v):
            continue
        d = abs(Fraction(float(v)) - q)
        key = (d, cb % 2)
        if best is None or key < best[0]:
            best = (key, cb)
    return best[1]


def bf16_value(bits) -> float:
    return float(_bf16_from_bits(int(bits)))
