"""Writes stacked_chain.npz: the oracle's run of the stacked decode workload.

The workload: 12 MoE layers of the full decode shape (H=5120, I=2560, 256
experts, top-8) over T=8 tokens, 3,072 expert records (layer l holds the
generated experts 256 l .. 256 l + 255), each layer preceded by a 5120 x 5120
affine8_g64 resident linear and a weightless RMSNorm (eps 1e-6), with the
residual added per layer:

    n_l  = rmsnorm(h_l)                      bf16
    a_l  = affine8_l(n_l)                    bf16, residents by the q8 rule
    e, w = top-8 of softmax(a_l . Wr_l)      router f32, one W_r per layer
    h_l+1 = bf16(h_l + sum_j w_j down(bf16(silu(gate a_l) * up a_l)))

Formats: "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
residents" ("What this pack holds": NVFP4 records and the global-scale rule;
the residents and q8-rule bullets for affine8_g64); FP32 router and SwiGLU
with BF16 mids per "Beam-1.0-501B-A23B VQ GGUF" ("What stays native").

Everything here comes from the seeded generators (synth) and the oracle; run
it from the repository root:  python tests/golden/make_stacked.py
Stored: per layer the oracle's router logits, its routing (idx, w), the gap
between the k-th and (k+1)-th logit of every token, and the bf16 state h_l+1;
the last layer's f32 output before rounding.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stacked_chain.npz")


def main():
    c = W.CONFIGS["stacked"]
    H, I, E, k, T, L = c["H"], c["I"], c["E"], c["k"], c["T"], c["layers"]
    seed, bseed = c["seed"], c["bank_seed"]
    h = synth.activations(seed, T, H)
    idx_all = np.zeros((L, T, k), np.int32)
    w_all = np.zeros((L, T, k), np.float32)
    gap_all = np.zeros((L, T), np.float32)
    lg_all = np.zeros((L, T, E), np.float32)
    h_all = np.zeros((L, T, H), np.uint16)
    y_last = None
    for l in range(L):
        t0 = time.time()
        n = oracle.rmsnorm(h, 1e-6)
        codes, scales, biases = oracle.q8_quantize(synth.resident_weights(seed, H, H, layer=l))
        _, a = oracle.affine8_linear(n, codes, scales, biases)
        logits = oracle.router_logits(a, synth.router_weights(seed, H, E, layer=l))
        idx, w = oracle.route_topk(logits, k)
        srt = np.sort(logits.astype(np.float64), axis=1)[:, ::-1]
        gap_all[l] = (srt[:, k - 1] - srt[:, k]).astype(np.float32)
        recs = {}
        for e in np.unique(idx):
            codes_e, scales_e, g_e = W.host_parts(bseed, l * E + int(e), H, I)
            recs[int(e)] = oracle.pack_record(H, I, codes_e, scales_e, g_e)
        yf, yb = oracle.moe_forward(recs, E, H, I, a, idx, w, residual=h)
        idx_all[l], w_all[l], h_all[l], lg_all[l] = idx, w, yb, logits
        h = yb
        y_last = yf
        print(f"layer {l}: {len(recs)} experts, min top-k gap {gap_all[l].min():.3e}, "
              f"rms {np.sqrt(np.mean(yf.astype(np.float64) ** 2)):.4f}, {time.time() - t0:.1f} s", flush=True)
    np.savez_compressed(OUT, idx=idx_all, w=w_all, gap=gap_all, logits=lg_all, h=h_all, y_last_f32=y_last)
    print("wrote", OUT, os.path.getsize(OUT), "bytes")


if __name__ == "__main__":
    main()
