"""The five layer workloads, built on a device from the seeded generators.

Shapes and value distributions are those of the five layer configs:
  tiny     H=256,  I=128,  E=16,  top-2, T=4,    router logits x . Wr
  decode   H=5120, I=2560, E=256, top-8, T=1,    router logits x . Wr
  batched  same layer, T=32,   logits N(0,1) + Zipf(1.1)-rank bias
  prefill  same layer, T=8192, logits N(0,1) + Zipf(1.1)-rank bias
  stacked  12 layers of the decode shape (3,072 records), T=8, each layer
           preceded by a 5120 x 5120 affine8_g64 resident linear
The three single-layer configs at the full shape share one bank (seed 1).
Banks are packed through the library's own pack entry point.
"""
import numpy as np
import torch

from . import activations, expert_parts, router_weights, skewed_logits, vq_codebook, vq_expert_parts

CONFIGS = {
    "tiny": dict(H=256, I=128, E=16, k=2, T=4, routing="router", seed=0, bank_seed=0),
    "decode": dict(H=5120, I=2560, E=256, k=8, T=1, routing="router", seed=1, bank_seed=1),
    "batched": dict(H=5120, I=2560, E=256, k=8, T=32, routing="zipf", seed=2, bank_seed=1),
    "prefill": dict(H=5120, I=2560, E=256, k=8, T=8192, routing="zipf", seed=3, bank_seed=1),
    "stacked": dict(H=5120, I=2560, E=256, k=8, T=8, layers=12, routing="router", seed=4, bank_seed=4),
}


def build_bank(seed, H, I, E, device="cuda", chunk=16, expert0=0):
    """A packed bank of E records whose expert e holds the seeded parts of expert
    id expert0 + e. Returns (descriptor, base tensor)."""
    import weight_quantized_moe_amd as wq

    bank, base = wq.alloc_bank(H, I, E, device)
    stride = bank.stride
    for e0 in range(0, E, chunk):
        n = min(chunk, E - e0)
        parts = [expert_parts(seed, expert0 + e0 + j, H, I, device) for j in range(n)]
        codes = [torch.stack([p[0][q] for p in parts]).contiguous() for q in range(3)]
        scales = [torch.stack([p[1][q] for p in parts]).contiguous() for q in range(3)]
        g = [torch.tensor(np.array([p[2][q] for p in parts]), dtype=torch.float32, device=device) for q in range(3)]
        sub = wq.moe_nvfp4_bank_init(base[e0 * stride:(e0 + n) * stride], H, I, n)
        wq.moe_pack_nvfp4_bank(sub, codes, scales, g)
        del parts, codes, scales, g
    torch.cuda.synchronize()
    return bank, base


def build_vq_bank(seed, H, I, E, device="cuda", chunk=16):
    """A packed bank of E 8-dim VQ records (expert e holds the seeded parts of
    expert e) over the seeded codebook. Returns (descriptor, base, codebook)."""
    import weight_quantized_moe_amd as wq

    cb = torch.from_numpy(vq_codebook(seed).reshape(-1).copy()).to(device)
    bank, base = wq.alloc_vq_bank(cb, H, I, E, device)
    stride = bank.stride
    for e0 in range(0, E, chunk):
        n = min(chunk, E - e0)
        parts = [vq_expert_parts(seed, e0 + j, H, I, device) for j in range(n)]
        idx = [torch.stack([p[0][q] for p in parts]).contiguous() for q in range(3)]
        gains = [torch.from_numpy(np.stack([p[1][q] for p in parts]).view(np.int16)).to(device) for q in range(3)]
        sub = wq.moe_vq_bank_init(base[e0 * stride:(e0 + n) * stride], cb, H, I, n)
        wq.moe_vq_pack_bank(sub, idx, gains)
        del parts, idx, gains
    torch.cuda.synchronize()
    return bank, base, cb


def host_parts(seed, expert, H, I):
    """Numpy parts of one expert (the same bytes the device generator makes)."""
    codes, scales, g = expert_parts(seed, expert, H, I, "cpu")
    return [c.numpy().view(np.uint32) for c in codes], [s.numpy() for s in scales], g


def inputs(name, variant=0):
    """Host inputs of a config: x bf16 bits [T][H], and either the router
    weights (f32 [E][H]) or the given logits (f32 [T][E]). `variant` draws a
    different x (and logits) from the same distribution."""
    c = CONFIGS[name]
    seed = c["seed"] + 1000 * variant
    x = activations(seed, c["T"], c["H"])
    if c["routing"] == "router":
        return x, router_weights(c["seed"], c["H"], c["E"]), None
    return x, None, skewed_logits(seed, c["T"], c["E"], rank_seed=c["seed"])
