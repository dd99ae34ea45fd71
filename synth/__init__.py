"""Seeded synthetic inputs for the NVFP4 MoE layer (tests, smoke check, benchmark).

This module holds none of the layer's arithmetic: it only draws inputs. Both the
HIP path and the CPU oracle receive the same arrays from here.

Randomness comes from one counter-based generator, SplitMix64 (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): value i
of stream s under seed S is mix64(key(S, s) + (i + 1) * 0x9E3779B97F4A7C15).
The integer draws (E2M1 code words, E4M3 scale bytes) are computed with
integer-only torch ops, so a CPU and a GPU produce identical bytes; float draws
(activations, router weights, logits, globals) are made on the host in f64 and
uploaded.

Value distributions (the workload descriptions of the five layer configs):
  * E2M1 codes uniform over 0..15, 8 per U32 word;
  * E4M3 block scales e4m3(|N(0,1)| * 0.05 + 1e-3), drawn exactly by comparing
    a 32-bit uniform with the cumulative probability of each E4M3 rounding
    interval (round to nearest);
  * globals g = 2688 * U(0.5, 2) in f32;
  * activations bf16 N(0,1); router weights f32 N(0, 0.02);
  * skewed router logits N(0,1) + r_e^(-1.1), r a seeded permutation of 1..E;
  * resident weights bf16 N(0, 0.02).
"""
import math

import numpy as np
import torch

GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# sub-stream ids (one per tensor kind); expert/projection indices are added
S_X, S_WR, S_LOGIT, S_PERM, S_G, S_AFF = 1, 2, 3, 4, 5, 6
S_CODES = 1 << 20
S_SCALES = 2 << 20
S_VQIDX = 3 << 20
S_VQGAIN, S_CB = 7, 8


def _signed(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for the vector forms)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def key(seed: int, stream: int) -> int:
    return mix64_int((seed * 0x100000001B3 + stream * GOLDEN + 0x632BE59BD9B4E019) & MASK64)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        return z ^ (z >> np.uint64(31))


def hash64_np(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key(seed, stream)) + i * np.uint64(GOLDEN)
    return _mix64_np(z)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """logical right shift of int64 bit patterns"""
    return (z >> s) & ((1 << (64 - s)) - 1)


def hash64_torch(seed: int, stream: int, start: int, n: int, device) -> torch.Tensor:
    """Same values as hash64_np, as int64 bit patterns (two's-complement wrap)."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = i * _signed(GOLDEN) + _signed(key(seed, stream))
    z = (z ^ _srl(z, 30)) * _signed(M1)
    z = (z ^ _srl(z, 27)) * _signed(M2)
    return z ^ _srl(z, 31)


def uniform01_np(seed, stream, n, start=0):
    """f64 uniforms in [0, 1) with 53 random bits"""
    h = hash64_np(seed, stream, start, n)
    return (h >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


def normal_np(seed, stream, n, start=0):
    """f64 N(0,1) by Box-Muller over pairs of uniforms"""
    m = (n + 1) // 2
    u = uniform01_np(seed, stream, 2 * m, 2 * start)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m)
    z[0::2] = r * np.cos(2.0 * math.pi * u2)
    z[1::2] = r * np.sin(2.0 * math.pi * u2)
    return z[:n]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """f64/f32 -> bf16 bit patterns (via f32, torch's round-to-nearest-even)"""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---- small float tensors (host) --------------------------------------------
def activations(seed, T, H, stream=S_X):
    """bf16 N(0,1) [T][H] as uint16 bits"""
    return to_bf16_bits(normal_np(seed, stream, T * H).reshape(T, H))


def router_weights(seed, H, E, layer=0):
    """f32 N(0, 0.02) [E][H] (one row per expert)"""
    return (normal_np(seed, S_WR + 16 * layer, H * E) * 0.02).astype(np.float32).reshape(E, H)


def zipf_ranks(seed, E, s=1.1):
    """per-expert bias r_e^(-s), r a seeded permutation of 1..E"""
    h = hash64_np(seed, S_PERM, 0, E)
    order = np.argsort(h, kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    return rank.astype(np.float64) ** (-s)


def skewed_logits(seed, T, E, s=1.1, rank_seed=None):
    """f32 router logits N(0,1) + Zipf-rank bias [T][E]; the expert ranks come
    from rank_seed (default: seed), the noise from seed"""
    z = normal_np(seed, S_LOGIT, T * E).reshape(T, E)
    r = zipf_ranks(seed if rank_seed is None else rank_seed, E, s)
    return (z + r[None, :]).astype(np.float32)


def global_scales(seed, n_records):
    """f32 g = 2688 * U(0.5, 2), [n_records][3] (gate, up, down)"""
    u = uniform01_np(seed, S_G, 3 * n_records)
    return (2688.0 * (0.5 + 1.5 * u)).astype(np.float32).reshape(n_records, 3)


def resident_weights(seed, N, K, layer=0):
    """bf16 N(0, 0.02) [N][K] as uint16 bits"""
    return to_bf16_bits((normal_np(seed, S_AFF + 16 * layer, N * K) * 0.02).reshape(N, K))


# ---- integer bank draws (host or device) -----------------------------------
_E4M3_THRESH = None


def e4m3_scale_thresholds() -> np.ndarray:
    """Cumulative 32-bit thresholds T_c, c = 0..125: a draw u (32-bit uniform)
    maps to the E4M3 byte #{c : T_c <= u}, which has the probability that
    round-to-nearest(|N(0,1)| * 0.05 + 1e-3) lands on that byte."""
    global _E4M3_THRESH
    if _E4M3_THRESH is None:
        vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        mids = 0.5 * (vals[:-1] + vals[1:])  # boundary between byte c and c+1
        z = np.maximum(mids - 1e-3, 0.0) / 0.05
        cdf = np.array([math.erf(v / math.sqrt(2.0)) for v in z])
        _E4M3_THRESH = np.minimum(np.round(cdf * 4294967296.0), 4294967296.0).astype(np.int64)
    return _E4M3_THRESH


def code_words(seed, stream, n_words, device="cpu", start_word=0) -> torch.Tensor:
    """n_words U32 words of uniform 4-bit codes (int32 bit patterns); word w is the
    low (even w) or high (odd w) half of hash (w // 2). start_word must be even."""
    assert start_word % 2 == 0
    nh = (n_words + 1) // 2
    h = hash64_torch(seed, stream, start_word // 2, nh, device)
    lo = h & 0xFFFFFFFF
    hi = _srl(h, 32)
    w = torch.stack([lo, hi], dim=1).reshape(-1)[:n_words]
    w = w - ((w >> 31) << 32)  # to the signed range, exactly
    return w.to(torch.int32)


def scale_bytes(seed, stream, n, device="cpu", start=0) -> torch.Tensor:
    """n E4M3 block-scale bytes (uint8)"""
    h = hash64_torch(seed, stream, start, n, device)
    u = _srl(h, 32)
    thr = torch.from_numpy(e4m3_scale_thresholds()).to(device)
    return torch.searchsorted(thr, u, right=True).to(torch.uint8)


def expert_parts(seed, expert, H, I, device="cpu"):
    """The 9 parts of one expert: codes[p] int32 [out][in/8], scales[p] uint8
    [out][in/16] (p = gate, up, down) and g[3] f32. Gate and up are [I][H],
    down is [H][I]."""
    codes, scales = [], []
    for p in range(3):
        out, inn = (H, I) if p == 2 else (I, H)
        codes.append(code_words(seed, S_CODES + 3 * expert + p, out * inn // 8, device).reshape(out, inn // 8))
        scales.append(scale_bytes(seed, S_SCALES + 3 * expert + p, out * inn // 16, device).reshape(out, inn // 16))
    g = expert_globals(seed, expert)
    return codes, scales, g


def expert_globals(seed, expert):
    """g (gate, up, down) of one expert: entries 3e..3e+2 of the globals stream"""
    u = uniform01_np(seed, S_G, 3, start=3 * expert)
    return (2688.0 * (0.5 + 1.5 * u)).astype(np.float32)


# ---- 8-dim VQ experts -------------------------------------------------------
def vq_codebook(seed, n=4096):
    """n codewords of 8 E4M3 bytes [n][8]: N(0,1) values rounded f32 -> f16 ->
    E4M3 (round to nearest even at each step)"""
    z = normal_np(seed, S_CB, 8 * n).astype(np.float32)
    h = z.astype(np.float16).astype(np.float32)
    return torch.from_numpy(h).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(n, 8)


def vq_expert_parts(seed, expert, H, I, device="cpu"):
    """idx[p]: uint8 packed 12-bit index rows [out][in * 3 / 16] (uniform
    indices: uniform bytes), gains[p]: f16 bits [out] of 0.02 * U(0.5, 2);
    p = gate, up, down (gate and up [I][H], down [H][I])."""
    idx, gains = [], []
    for p in range(3):
        out, inn = (H, I) if p == 2 else (I, H)
        nbytes = out * inn * 3 // 16
        w = code_words(seed, S_VQIDX + 3 * expert + p, nbytes // 4, device)
        idx.append(w.view(torch.uint8).reshape(out, inn * 3 // 16))
        u = uniform01_np(seed, S_VQGAIN, out, start=(3 * expert + p) << 16)
        gains.append((0.02 * (0.5 + 1.5 * u)).astype(np.float16).view(np.uint16))
    return idx, gains
