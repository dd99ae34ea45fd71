"""Benchmark of the NVFP4 MoE layer on one MI355X.

One step = the whole hot path on one batch: router logits + top-k (S1, S2),
pair sort (S3), gate/up + SwiGLU (S4, S5), down (S6) and the weighted combine
(S7), all through the C ABI, inputs resident in HBM. The decode step is one
moe_nvfp4_layer call (router and top-k inside the gate/up launch); with
--two-call it is moe_route_topk followed by moe_nvfp4_forward.

Headline (value): decode, T=1, H=5120, I=2560, 256 experts, top-8, as HBM
GB/s of algorithmic bytes (the 8 selected records of 22,118,412 B + the f32
router 5,242,880 B + x and y). Consecutive steps rotate over 64 different
activations, so the routed records change every step and the 256 MB
Infinity Cache cannot serve them.
Second leg (prefill): T=8192 with Zipf(1.1)-skewed logits given, as TFLOP/s of
2 * 65,536 * 3 * 5120 * 2560 flop.
roofline: the dominant kernel of each leg, its algorithmic bytes (flop) per
launch over its mean launch time from HIP events recorded around each launch
on the stream it runs on.
step_us: median, p10 and p90 of per-step times (a separate pass with an event
after every step). status: the workspace's status word after the timed
passes (0, or the run stops: a routing wait that gave up or an expert id
outside the bank would make the outputs invalid).
peak_probes / roofline.peak_measured: what this GPU reaches in practice, a
streaming read of HBM (1 GiB, and pieces of the decode step's 182 MB read in
turn from a 4 GiB buffer) and a bf16 MFMA loop (moe_probe_*), reported beside
the data-sheet peaks.
cpu_baseline: the CPU oracle (as is) on a bounded sample of the decode
workload, on this host's cores; `extra` times the tiny and decode workloads
on one thread, the batched T=32 workload in full and the prefill workload on
a 64-token sample (extrapolated to 8192 tokens).

roofline.traffic: HBM bytes per launch of the dominant decode kernel, from
rocprofv3 FETCH_SIZE + WRITE_SIZE counter runs scaled by what the same
counters read for a plain device copy of known size; read from
profiles/traffic_decode_gateup.txt and reported only while the kernel source
it was measured on is unchanged (its SHA-1 is recorded there), else null.

Expert cache leg (--only cache, not part of the default run): the bank in
pinned host memory, a bounded pool of HBM slots (moe_cache_*), single-token
decode steps on Zipf(1.1)-skewed routing; reports the host-to-HBM copy rate
on an all-miss pattern against PCIe 5.0 x16 (64 GB/s per direction), and per
pool size the hit rate and the time per step (prepare + forward).

VQ leg (--only vq, not part of the default run): the same single-token decode
step over the 8-dim VQ expert format (256 records of 7,393,280 B, 12-bit
indices, a 32 KiB E4M3 codebook): moe_route_topk (router + top-k) then
moe_vq_forward, as GB/s of algorithmic bytes (8 VQ records + the f32 router +
the codebook + x and y).

Verify leg (--only verify, not part of the default run): the one-call layer
(moe_nvfp4_layer: router, top-k, experts, combine) on T = 1..4 tokens, the
draft-verify shape; GB/s over the distinct selected records + W_r + x, y.

Residents leg (--only affine8, not part of the default run): the 5120 x 5120
affine8_g64 resident linear at T = 256, 1,024 and 8,192 tokens (the MFMA GEMM
path), as TFLOP/s of 2 T K N against 2.5 PFLOP/s.

Batched leg (--only batched): T = 32 tokens on Zipf(1.1)-skewed logits
(given), moe_route_topk + moe_nvfp4_forward, GB/s over the distinct selected
records + x, y. Stacked leg (--only stacked): 12 layers of the decode shape,
each RMSNorm + a 5120 x 5120 affine8_g64 resident + the one-call layer with
the residual, T = 8; GB/s over the residents, routers and distinct records of
all 12 layers (about 15.6 GB per step).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--prefill-steps P]
       [--only decode|prefill|cache|vq|verify|affine8|batched|stacked|peak] [--no-cpu-baseline]
       [--no-probes] [--two-call]
Profiling helpers: --copy-calibration (device copies of 1 GiB, for the
counter scale factor); --summarize-pmc DIR (per-kernel mean counter values
per dispatch from a rocprofv3 --pmc output directory; no GPU needed).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import weight_quantized_moe_amd as wq  # noqa: E402
from synth import workloads as W  # noqa: E402

METRIC = "NVFP4 MoE layer: decode HBM GB/s (T=1) + prefill TFLOP/s (T=8192), 1 GPU"
HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 64.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def kernel_avg_ms(name):
    ms, n = wq.moe_profile_read(name)
    return (ms / n if n else float("nan")), n


class DecodeLeg:
    def __init__(self, bank):
        c = W.CONFIGS["decode"]
        self.c, self.bank = c, bank
        H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], c["T"]
        xs = [W.inputs("decode", v)[0] for v in range(ROTATE)]
        _, Wr, _ = W.inputs("decode")
        self.x = bf16_dev(np.stack(xs))  # [ROTATE][T][H]
        self.Wr = torch.from_numpy(Wr).cuda()
        self.logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        self.idx = torch.empty((ROTATE, T, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((ROTATE, T, k), dtype=torch.float32, device="cuda")
        self.y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
        self.i = 0
        self.two_call = False

    def step(self):
        c, r = self.c, self.i % ROTATE
        self.i += 1
        if self.two_call:
            wq.moe_route_topk(self.x[r], self.Wr, self.logits, c["T"], c["H"], c["E"], c["k"], self.idx[r],
                              self.w[r])
            wq.moe_nvfp4_forward(self.bank, self.x[r], c["T"], self.idx[r], self.w[r], c["k"], None, self.y, 0,
                                 self.ws)
        else:
            wq.moe_nvfp4_layer(self.bank, self.x[r], self.Wr, c["T"], c["k"], None, self.logits, self.idx[r],
                               self.w[r], self.y, 0, self.ws)

    def step_bytes(self, r):
        """algorithmic HBM bytes of the step that used activation r"""
        c = self.c
        n_unique = len(np.unique(self.idx_host[r]))
        rec = wq.moe_nvfp4_record_bytes(c["H"], c["I"])
        return n_unique * rec + c["H"] * c["E"] * 4 + 2 * c["T"] * c["H"] * 2

    def gateup_bytes(self, r):
        """algorithmic bytes of the gate/up launch: gate and up of the selected
        records, x, the bf16 mids written; in the one-call layer also the f32
        router weights and the logits, idx and w written"""
        c = self.c
        n_unique = len(np.unique(self.idx_host[r]))
        per_proj = c["H"] * c["I"] // 2 + c["H"] * c["I"] // 16
        b = n_unique * 2 * per_proj + c["T"] * c["H"] * 2 + len(self.idx_host[r].ravel()) * c["I"] * 2
        if not self.two_call:
            b += c["H"] * c["E"] * 4 + c["T"] * (c["E"] + 2 * c["k"]) * 4
        return b


class PrefillLeg:
    def __init__(self, bank):
        c = W.CONFIGS["prefill"]
        self.c, self.bank = c, bank
        H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], c["T"]
        x, _, logits = W.inputs("prefill")
        self.x = bf16_dev(x)
        self.logits = torch.from_numpy(logits).cuda()
        self.idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
        self.flop = 2 * T * k * 3 * H * I

    def step(self):
        c = self.c
        wq.moe_route_topk(None, None, self.logits, c["T"], c["H"], c["E"], c["k"], self.idx, self.w)
        wq.moe_nvfp4_forward(self.bank, self.x, c["T"], self.idx, self.w, c["k"], None, self.y, 0, self.ws)


def timed(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3


def step_stats(fn, steps):
    """Per-step times (us) from an event recorded after every step on the
    stream (a pass of its own: the events cost a little): median, p10, p90."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(s)
    for i in range(steps):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)])
    return {"median": round(float(np.median(d)), 2), "p10": round(float(np.percentile(d, 10)), 2),
            "p90": round(float(np.percentile(d, 90)), 2), "steps": steps}


def check_status(ws, what):
    """The layer's workspace status word after the timed passes: 0, or the run
    is invalid (a routing wait that gave up, an expert outside the bank)."""
    st = wq.moe_status_read(ws)
    if st != 0:
        raise SystemExit(f"{what}: workspace status word {st:#x} after the timed passes: outputs invalid")
    return st


def probe_peaks(fast=False):
    """What this GPU reaches in practice: a streaming read of HBM (1 GiB, and
    pieces of the decode step's size read in turn from a 4 GiB buffer, so the
    256 MB Infinity Cache cannot serve them) and a bf16 MFMA loop in
    back-to-back bursts of a few ms (the clock settles as under the prefill)."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()

    def time_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev0.record(s)
        for r in range(reps):
            fn(r)
        ev1.record(s)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    GiB = 1 << 30
    rows = []
    configs = [(v, b) for v in range(4) for b in ((2048, 8192) if fast else (1024, 2048, 4096, 8192))]
    for v, b in configs:
        ms = time_ms(lambda r=0: wq.moe_probe_hbm_read(buf[(r % 3) * GiB:], GiB, v, b, sink), 6)
        rows.append({"variant": v, "blocks": b, "GBps": round(GiB / (ms * 1e-3) / 1e9, 1)})
    best = max(rows, key=lambda r: r["GBps"])
    piece = 182210656 // 16 * 16
    n_pieces = (4 * GiB) // piece
    ms = time_ms(lambda r=0: wq.moe_probe_hbm_read(buf[(r % n_pieces) * piece:], piece, best["variant"],
                                                   best["blocks"], sink), 64)
    piece_gbs = piece / (ms * 1e-3) / 1e9
    del buf
    fsink = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    blocks, iters = 2048, 4000
    flop = blocks * 4 * 4 * iters * 32768
    ms = time_ms(lambda r=0: wq.moe_probe_mfma_bf16(blocks, iters, fsink), 10)
    mfma_tf = flop / (ms * 1e-3) / 1e12
    log(f"probes: HBM read 1 GiB {best['GBps']:.0f} GB/s (variant {best['variant']}, {best['blocks']} blocks), "
        f"{piece / 1e6:.0f} MB pieces {piece_gbs:.0f} GB/s; bf16 MFMA loop {mfma_tf:.0f} TFLOP/s ({ms:.2f} ms bursts)")
    return {"hbm_read_1GiB_GBps": best["GBps"], "hbm_read_step_size_GBps": round(piece_gbs, 1),
            "hbm_read_best": {"variant": best["variant"], "blocks": best["blocks"]},
            "hbm_read_sweep": rows, "mfma_bf16_TFLOPs": round(mfma_tf, 1),
            "mfma_burst_ms": round(ms, 3),
            "note": "streaming read: 16-byte loads, grid-stride; MFMA: v_mfma_f32_32x32x16_bf16, register "
                    "operands, 2048 workgroups of 4 waves, back-to-back bursts"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_gateup.txt")
DECODE_SRC = os.path.join(ROOT, "weight_quantized_moe_amd", "csrc", "decode.hip")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_T8192_counters.txt")
PREFILL_SRC = os.path.join(ROOT, "weight_quantized_moe_amd", "csrc", "prefill.hip")


def recorded_traffic(name, path=TRAFFIC_FILE, source=DECODE_SRC):
    """Bytes per launch of launch `name` from a committed counter summary, if
    it was measured on that launch and the current kernel source; else None."""
    try:
        fields = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
        src = hashlib.sha1(open(source, "rb").read()).hexdigest()
        if fields.get("source_sha1", "").strip() != src or fields.get("launch", "").strip() != name:
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(nbytes=1 << 30, reps=5):
    """Plain device copies of nbytes, for scaling FETCH_SIZE / WRITE_SIZE."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def summarize_pmc(d):
    """Mean counter value per dispatch and kernel over rocprofv3 counter CSVs."""
    agg, disp = {}, {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            key = (k, r["Counter_Name"])
            agg[key] = agg.get(key, 0.0) + float(r["Counter_Value"])
            disp.setdefault(k, set()).add(r["Dispatch_Id"])
    for (k, cname), v in sorted(agg.items()):
        print(f"{k[:70]:70s} {cname:12s} dispatches={len(disp[k]):4d} mean_per_dispatch={v / len(disp[k]):.6g}")


def _omp_threads(n):
    """Sets the OpenMP thread count of the oracle's parallel loops (libgomp's
    own setter, on this thread); returns the previous count."""
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    prev = gomp.omp_get_max_threads()
    gomp.omp_set_num_threads(int(n))
    return prev


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c, budget_s=20.0):
    """The oracle, as it stands, timed on this host: the headline is the decode
    workload (router + top-k + layer, T=1) on all OpenMP threads, as many
    steps as fit the budget (1 to 8). `extra` times the other layer workloads:
    tiny and decode on one thread, batched T=32 in full, and prefill on a
    seeded sample of 64 tokens (512 pairs) with the full layer extrapolated
    linearly in tokens. Records are generated once (not timed)."""
    import oracle

    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    threads = _omp_threads(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    _omp_threads(threads)
    rec_bytes = wq.moe_nvfp4_record_bytes(H, I)
    t_gen = time.perf_counter()
    cache = {}

    def records(experts):
        for e in experts:
            if int(e) not in cache:
                cc, ss, gg = W.host_parts(c["bank_seed"], int(e), H, I)
                cache[int(e)] = oracle.pack_record(H, I, cc, ss, gg)
        return {int(e): cache[int(e)] for e in experts}

    def decode_step(x, Wr):
        idx_probe, _ = oracle.route_topk(oracle.router_logits(x, Wr), k)
        recs = records(np.unique(idx_probe))
        t0 = time.perf_counter()
        lg = oracle.router_logits(x, Wr)
        idx, w = oracle.route_topk(lg, k)
        oracle.moe_forward(recs, E, H, I, x, idx, w)
        dt = time.perf_counter() - t0
        return dt, len(np.unique(idx)) * rec_bytes + H * E * 4 + 2 * H * 2

    _, Wr, _ = W.inputs("decode")
    t_total, n, nbytes = 0.0, 0, 0
    while n == 0 or t_total < budget_s:
        dt, nb = decode_step(W.inputs("decode", n % ROTATE)[0], Wr)
        t_total += dt
        nbytes += nb
        n += 1
        if n >= 8:
            break
    out = {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": f"{n} decode steps (T=1, router + top-8 + layer), {t_total:.1f} s, f64-accumulating C oracle"}
    extra = {}
    # decode and tiny on one thread
    _omp_threads(1)
    dt, nb = decode_step(W.inputs("decode", 0)[0], Wr)
    extra["decode_1thread"] = {"GBps": round(nb / dt / 1e9, 4), "s": round(dt, 2), "steps": 1}
    ct = W.CONFIGS["tiny"]
    xt, Wrt, _ = W.inputs("tiny")
    rt = {}
    for e in range(ct["E"]):
        cc, ss, gg = W.host_parts(ct["bank_seed"], e, ct["H"], ct["I"])
        rt[e] = oracle.pack_record(ct["H"], ct["I"], cc, ss, gg)
    for thr in (1, threads):
        _omp_threads(thr)
        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            lgt = oracle.router_logits(xt, Wrt)
            it, wt = oracle.route_topk(lgt, ct["k"])
            oracle.moe_forward(rt, ct["E"], ct["H"], ct["I"], xt, it, wt)
        dt = (time.perf_counter() - t0) / reps
        extra[f"tiny_{thr}thread"] = {"ms_per_step": round(dt * 1e3, 3), "steps": reps}
    _omp_threads(threads)
    # batched T=32 in full (logits given)
    cb = W.CONFIGS["batched"]
    xb, _, lgb = W.inputs("batched")
    ib, wb = oracle.route_topk(lgb, k)
    recs = records(np.unique(ib))
    t0 = time.perf_counter()
    ib, wb = oracle.route_topk(lgb, k)
    oracle.moe_forward(recs, E, H, I, xb, ib, wb)
    dt = time.perf_counter() - t0
    nb = len(np.unique(ib)) * rec_bytes + 2 * cb["T"] * H * 2
    extra["batched_T32"] = {"GBps": round(nb / dt / 1e9, 4), "s": round(dt, 2), "distinct_records": len(np.unique(ib))}
    # prefill: top-k of all 8192 tokens, the layer on a seeded sample of 64
    cp = W.CONFIGS["prefill"]
    xp, _, lgp = W.inputs("prefill")
    sample = np.sort(np.random.default_rng(cp["seed"]).choice(cp["T"], 64, replace=False))
    ip_all, wp_all = oracle.route_topk(lgp, k)
    recs = records(np.unique(ip_all[sample]))
    t0 = time.perf_counter()
    ip_all, wp_all = oracle.route_topk(lgp, k)
    oracle.moe_forward(recs, E, H, I, xp[sample], ip_all[sample], wp_all[sample])
    dt = time.perf_counter() - t0
    flop = 2 * len(sample) * k * 3 * H * I
    full_s = dt * cp["T"] / len(sample)
    extra["prefill_sample"] = {"tokens": len(sample), "pairs": len(sample) * k, "s": round(dt, 2),
                               "TFLOPs": round(flop / dt / 1e12, 6), "full_layer_s_extrapolated": round(full_s, 1),
                               "basis": "sample time x 8192 / 64 (tokens); the sample's expert dequant is "
                                        "counted once, so this overstates the full layer slightly"}
    extra["wall_s_with_record_generation"] = round(time.perf_counter() - t_gen, 1)
    out["extra"] = extra
    return out


def prefill_leg(bank, P, peaks=None):
    pre = PrefillLeg(bank)
    pms, _ = timed(pre.step, P, 2)
    tflops = pre.flop / (pms / P * 1e-3) / 1e12
    status = check_status(pre.ws, "prefill")
    dist = step_stats(pre.step, P)
    wq.moe_profile_enable(True)
    for _ in range(P):
        pre.step()
    torch.cuda.synchronize()
    pk = {n_: kernel_avg_ms(n_) for n_ in ["topk", "sort", "sort_count", "sort_scan", "sort_place", "prefill_gateup", "prefill_down", "combine"]}
    pk = {n_: v for n_, v in pk.items() if v[1]}
    wq.moe_profile_enable(False)
    for n_, (avg, cnt) in pk.items():
        log(f"  {n_:15s} {avg * 1e3:8.2f} us x {cnt}")
    gu_flop = 2 * pre.c["T"] * pre.c["k"] * 2 * pre.c["H"] * pre.c["I"]
    gu_tf = gu_flop / (pk["prefill_gateup"][0] * 1e-3) / 1e12
    log(f"prefill: {pms / P:.3f} ms/step, {tflops:.1f} TFLOP/s")
    roof_extra = {}
    if peaks:
        pm = peaks["mfma_bf16_TFLOPs"]
        roof_extra = {"peak_measured": pm, "frac_measured": round(gu_tf / pm, 4),
                      "peak_measured_by": "bf16 MFMA loop (moe_probe_mfma_bf16)"}
    return {"value": round(tflops, 2), "unit": "TFLOP/s", "steps": P, "ms_per_step": round(pms / P, 4),
            "step_us": dist, "status": status,
            "workload": "prefill: T=8192, top-8 of 256 on Zipf(1.1)-skewed logits (given), "
                        "65,536 pairs, 5.154 TFLOP per step",
            "roofline": {"kernel": "prefill_gateup", "bound": "mfma", "achieved": round(gu_tf, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gu_tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("prefill_gateup", PREFILL_TRAFFIC_FILE, PREFILL_SRC),
                         "flop_per_launch": gu_flop,
                         "avg_launch_ms": round(pk["prefill_gateup"][0], 4), **roof_extra},
            "kernels_us": {n_: round(v[0] * 1e3, 2) for n_, v in pk.items()}}


def resident_parts(seed, N, K, layer=0):
    """codes, scales and biases of an affine8_g64 resident from the seeded bf16
    weights (scale and bias from each group's range; uniform codes: the values
    do not change the timing), built with torch alone"""
    w = synth.resident_weights(seed, N, K, layer=layer)
    wt = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16).float().view(N, K // 64, 64)
    lo, hi = wt.amin(dim=2), wt.amax(dim=2)
    scale = ((hi - lo) / 255.0).to(torch.bfloat16).view(torch.int16).contiguous()
    bias = lo.to(torch.bfloat16).view(torch.int16).contiguous()
    g = torch.Generator("cuda").manual_seed(1000 * seed + layer)
    codes = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=g).view(torch.int32)
    return codes.contiguous(), scale, bias


def batched_leg(bank, K, Wm):
    c = W.CONFIGS["batched"]
    H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], c["T"]
    nv = 8
    xs = bf16_dev(np.stack([W.inputs("batched", v)[0] for v in range(nv)]))
    lgs = torch.from_numpy(np.stack([W.inputs("batched", v)[2] for v in range(nv)])).cuda()
    idx = torch.empty((nv, T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((nv, T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
    state = {"i": 0}

    def step():
        r = state["i"] % nv
        state["i"] += 1
        wq.moe_route_topk(None, None, lgs[r], T, H, E, k, idx[r], w[r])
        wq.moe_nvfp4_forward(bank, xs[r], T, idx[r], w[r], k, None, y, 0, ws)

    ms_total, _ = timed(step, K, Wm)
    idx_h = idx.cpu().numpy()
    rec = wq.moe_nvfp4_record_bytes(H, I)
    rs = [(Wm + i) % nv for i in range(K)]
    nb = np.array([len(np.unique(idx_h[r])) * rec + 2 * T * H * 2 for r in rs], dtype=np.float64)
    gbs = nb.sum() / (ms_total * 1e-3) / 1e9
    log(f"batched T=32: {ms_total / K:.3f} ms/step, {gbs:.1f} GB/s, {nb.mean() / rec:.1f} distinct records")
    return {"workload": "T=32, top-8 of 256 on Zipf(1.1)-skewed logits (given), H=5120, I=2560", "steps": K,
            "ms_per_step": round(ms_total / K, 4), "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_step": int(nb.mean()), "distinct_records": round(float(nb.mean()) / rec, 1)}


def stacked_leg(K, Wm):
    c = W.CONFIGS["stacked"]
    H, I, E, k, T, L = c["H"], c["I"], c["E"], c["k"], c["T"], c["layers"]
    log(f"building the stacked banks: {L} x {E} records")
    banks = [W.build_bank(c["bank_seed"], H, I, E, expert0=l * E)[0] for l in range(L)]
    res = [resident_parts(c["seed"], H, H, layer=l) for l in range(L)]
    wrs = [torch.from_numpy(synth.router_weights(c["seed"], H, E, layer=l)).cuda() for l in range(L)]
    nv = 4
    h0s = bf16_dev(np.stack([synth.activations(c["seed"] + 1000 * v, T, H) for v in range(nv)]))
    hs = [torch.empty((T, H), dtype=torch.int16, device="cuda") for _ in range(2)]
    nrm = torch.empty((T, H), dtype=torch.int16, device="cuda")
    a = torch.empty((T, H), dtype=torch.int16, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
    uniq = []
    state = {"i": 0}

    def step():
        h = h0s[state["i"] % nv]
        state["i"] += 1
        for l in range(L):
            wq.moe_rmsnorm(h, T, H, 1e-6, nrm)
            codes, scale, bias = res[l]
            wq.affine8_g64_linear(nrm, codes, scale, bias, T, H, H, a)
            out = hs[l % 2]
            wq.moe_nvfp4_layer(banks[l], a, wrs[l], T, k, h, logits, idx[l], w[l], out, 0, ws)
            h = out

    ms_total, _ = timed(step, K, Wm)
    idx_h = idx.cpu().numpy()
    rec = wq.moe_nvfp4_record_bytes(H, I)
    per_layer_fixed = H * H + 2 * 2 * H * (H // 64) + H * E * 4 + 3 * T * H * 2
    nb = sum(len(np.unique(idx_h[l])) * rec for l in range(L)) + L * per_layer_fixed
    gbs = nb / (ms_total / K * 1e-3) / 1e9
    log(f"stacked 12 x T=8: {ms_total / K:.3f} ms/step, {gbs:.1f} GB/s (last step {nb / 1e9:.2f} GB)")
    return {"workload": "12 layers x (RMSNorm + 5120x5120 affine8_g64 + one-call NVFP4 layer with residual), T=8, "
                        "3,072 records (68 GB)", "steps": K, "ms_per_step": round(ms_total / K, 4),
            "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_step_last": int(nb), "note": "bytes counted from the last timed step's routing"}


def affine8_leg(K=5120, N=5120, steps=20, warm=3):
    w = synth.resident_weights(16, N, K)
    # codes, scales and biases of a 5120 x 5120 resident: the seeded bf16
    # weights through the library-independent q8 draw below (uniform codes,
    # scale and bias from the weight rows' range) keep the run free of the oracle
    wt = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16).float().view(N, K // 64, 64)
    lo, hi = wt.amin(dim=2), wt.amax(dim=2)
    scale = ((hi - lo) / 255.0).to(torch.bfloat16)
    bias = lo.to(torch.bfloat16)
    codes = torch.randint(0, 256, (N, K), dtype=torch.uint8, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    codes32 = codes.view(torch.int32).contiguous()
    rows = []
    for T in (256, 1024, 8192):
        x = bf16_dev(synth.activations(19, T, K))
        y = torch.empty((T, N), dtype=torch.int16, device="cuda")

        def step():
            wq.affine8_g64_linear(x, codes32, scale.view(torch.int16), bias.view(torch.int16), T, K, N, y)

        ms_total, _ = timed(step, steps, warm)
        tf = 2.0 * T * K * N / (ms_total / steps * 1e-3) / 1e12
        rows.append({"T": T, "ms": round(ms_total / steps, 4), "TFLOPs": round(tf, 1),
                     "frac_of_2.5PF": round(tf / BF16_PEAK_TFLOPS, 4)})
        log(f"affine8 T={T}: {ms_total / steps:.3f} ms, {tf:.1f} TFLOP/s")
    return {"workload": "affine8_g64 resident linear, K = N = 5120, bf16 activations", "rows": rows}


def verify_leg(bank, K, Wm):
    c = W.CONFIGS["decode"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    _, Wr, _ = W.inputs("decode")
    Wr = torch.from_numpy(Wr).cuda()
    rec = wq.moe_nvfp4_record_bytes(H, I)
    rows = []
    for T in (1, 2, 3, 4):
        xs = bf16_dev(np.stack([synth.activations(100 + v, T, H) for v in range(ROTATE)]))
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        idx = torch.empty((ROTATE, T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((ROTATE, T, k), dtype=torch.float32, device="cuda")
        y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
        state = {"i": 0}

        def step():
            r = state["i"] % ROTATE
            state["i"] += 1
            wq.moe_nvfp4_layer(bank, xs[r], Wr, T, k, None, logits, idx[r], w[r], y, 0, ws)

        ms_total, _ = timed(step, K, Wm)
        idx_h = idx.cpu().numpy()
        rs = [(Wm + i) % ROTATE for i in range(K)]
        nb = np.array([len(np.unique(idx_h[r])) * rec + H * E * 4 + 2 * T * H * 2 for r in rs], dtype=np.float64)
        gbs = nb.sum() / (ms_total * 1e-3) / 1e9
        row = {"T": T, "us_per_step": round(ms_total / K * 1e3, 2), "GBps": round(gbs, 1),
               "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4), "distinct_experts": round(float(nb.mean() - H * E * 4) / rec, 2)}
        rows.append(row)
        log(f"verify T={T}: {ms_total / K * 1e3:.1f} us/step, {gbs:.1f} GB/s")
    return {"workload": "one-call layer on T = 1..4 tokens (router f32, top-8 of 256, H=5120, I=2560), "
                        "64 rotating activations", "rows": rows}


def vq_leg(K, Wm):
    c = W.CONFIGS["decode"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    bank, base, cb = W.build_vq_bank(32, H, I, E)
    xs = bf16_dev(np.stack([W.inputs("decode", v)[0] for v in range(ROTATE)]))
    _, Wr, _ = W.inputs("decode")
    Wr = torch.from_numpy(Wr).cuda()
    logits = torch.empty((1, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((ROTATE, 1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((ROTATE, 1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.int16, device="cuda")
    ws = wq.workspace(wq.moe_vq_workspace_bytes(1, k, H, I))
    state = {"i": 0}

    def step():
        r = state["i"] % ROTATE
        state["i"] += 1
        wq.moe_route_topk(xs[r], Wr, logits, 1, H, E, k, idx[r], w[r])
        wq.moe_vq_forward(bank, xs[r], 1, idx[r], w[r], k, None, y, 0, ws)

    ms_total, _ = timed(step, K, Wm)
    idx_h = idx.cpu().numpy()
    rs = [(Wm + i) % ROTATE for i in range(K)]
    rec = wq.moe_vq_record_bytes(H, I)
    nb = np.array([len(np.unique(idx_h[r])) * rec + H * E * 4 + 32768 + 2 * H * 2 for r in rs], dtype=np.float64)
    gbs = nb.sum() / (ms_total * 1e-3) / 1e9
    wq.moe_profile_enable(True)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name in ["router", "topk", "vq_gateup", "vq_down"]:
        avg, cnt = kernel_avg_ms(name)
        if cnt:
            kern[name] = round(avg * 1e3, 2)
    wq.moe_profile_enable(False)
    gu_bytes = np.mean([len(np.unique(idx_h[r])) * 2 * I * (H * 3 // 16 + 2) for r in rs]) + 32768 + H * 2 + k * I * 2
    gu_gbs = gu_bytes / (kern["vq_gateup"] * 1e-6) / 1e9
    log(f"vq decode: {ms_total / K * 1e3:.1f} us/step, {gbs:.1f} GB/s; kernels {kern}")
    return {"value": round(gbs, 2), "unit": "GB/s", "steps": K, "us_per_step": round(ms_total / K * 1e3, 2),
            "workload": "decode T=1 over 8-dim VQ records (12-bit indices, 32 KiB E4M3 codebook), H=5120, I=2560, "
                        "256 experts, top-8; router f32; 64 rotating activations",
            "bytes_per_step": int(nb.mean()),
            "roofline": {"kernel": "vq_gateup", "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": int(gu_bytes),
                         "avg_launch_us": kern["vq_gateup"]},
            "kernels_us": kern}


def cache_leg(bank, base, pools=(32, 64, 128, 192), steps=256, warm=64):
    c = W.CONFIGS["decode"]
    E, k, H = c["E"], c["k"], c["H"]
    host_mem = torch.empty(base.numel(), dtype=torch.uint8, pin_memory=True)
    host_mem.copy_(base)
    hb = wq.moe_nvfp4_bank()
    hb.H, hb.I, hb.E, hb.record_bytes, hb.stride = bank.H, bank.I, bank.E, bank.record_bytes, bank.stride
    for i in range(9):
        hb.part_off[i] = bank.part_off[i]
    hb.base = host_mem.data_ptr()
    stride = bank.stride
    # routing of `steps + warm` single-token steps on Zipf-skewed logits (the
    # library's top-k)
    n_tok = steps + warm
    logits = torch.from_numpy(synth.skewed_logits(77, n_tok, E, rank_seed=c["seed"])).cuda()
    idx_d = torch.empty((n_tok, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((n_tok, k), dtype=torch.float32, device="cuda")
    wq.moe_route_topk(None, None, logits, n_tok, H, E, k, idx_d, w_d)
    idx_h = idx_d.cpu().numpy()
    xs = bf16_dev(np.stack([W.inputs("decode", v)[0] for v in range(8)]))
    y = torch.empty((1, H), dtype=torch.int16, device="cuda")

    def pool(n):
        mem = torch.empty(n * stride + 4096, dtype=torch.uint8, device="cuda")
        off = (-mem.data_ptr()) % 4096
        return mem, mem[off:off + n * stride]

    out = {"workload": "single-token decode steps, top-8 of 256 on Zipf(1.1)-skewed logits, the 256-record bank "
                       "in pinned host memory, a pool of HBM slots"}
    # host -> HBM rate: 8 slots, every step names 8 experts not resident
    mem, sb = pool(8)
    cache = wq.moe_cache_create(hb, sb, 8)
    reps = 64
    torch.cuda.synchronize()
    t0 = time.time()
    for r in range(reps):
        wq.moe_cache_prepare(cache, [(8 * r + j) % E for j in range(8)])
    torch.cuda.synchronize()
    dt = time.time() - t0
    _, _, nbytes = wq.moe_cache_stats(cache)
    wq.moe_cache_destroy(cache)
    del mem, sb
    gbs = nbytes / dt / 1e9
    out["h2d"] = {"GBps": round(gbs, 2), "peak": PCIE_PEAK_GBS, "frac": round(gbs / PCIE_PEAK_GBS, 4),
                  "bytes": int(nbytes), "records": reps * 8}
    log(f"cache: host->HBM {gbs:.1f} GB/s over {reps * 8} records")
    # decode through pools of several sizes
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(1, k, H, c["I"], E))
    rows = []
    for n in pools:
        mem, sb = pool(n)
        cache = wq.moe_cache_create(hb, sb, n)
        cb = wq.moe_cache_bank(cache)
        sidx = torch.empty((1, k), dtype=torch.int32, device="cuda")

        def step(t):
            ids = list(dict.fromkeys(int(e) for e in idx_h[t]))
            slot_of = wq.moe_cache_prepare(cache, ids)
            remap = dict(zip(ids, slot_of.tolist()))
            sidx.copy_(torch.tensor([[remap[int(e)] for e in idx_h[t]]], dtype=torch.int32), non_blocking=False)
            wq.moe_nvfp4_forward(cb, xs[t % 8], 1, sidx, w_d[t:t + 1], k, None, y, 0, ws)

        for t in range(warm):
            step(t)
        torch.cuda.synchronize()
        h0, m0, b0 = wq.moe_cache_stats(cache)
        t0 = time.time()
        for t in range(warm, warm + steps):
            step(t)
        torch.cuda.synchronize()
        dt = time.time() - t0
        h1, m1, b1 = wq.moe_cache_stats(cache)
        wq.moe_cache_destroy(cache)
        del mem, sb
        hit = (h1 - h0) / max(1, (h1 - h0) + (m1 - m0))
        row = {"slots": n, "hit_rate": round(hit, 4), "ms_per_step": round(dt / steps * 1e3, 4),
               "copied_MB_per_step": round((b1 - b0) / steps / 1e6, 2)}
        rows.append(row)
        log(f"cache: {n} slots, hit rate {hit:.3f}, {dt / steps * 1e3:.3f} ms/step")
    out["decode"] = rows
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "cache", "vq", "verify", "affine8", "batched",
                                       "stacked", "peak"])
    ap.add_argument("--no-probes", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--two-call", action="store_true",
                    help="decode step as moe_route_topk + moe_nvfp4_forward instead of moe_nvfp4_layer")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.only == "decode":
        args.no_prefill = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer runs on one MI355X; --gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wq.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.only == "peak":
        print(json.dumps({"peak": probe_peaks()}), flush=True)
        return
    if args.only == "vq":
        print(json.dumps({"vq": vq_leg(args.steps, args.warmup)}), flush=True)
        return
    if args.only == "affine8":
        print(json.dumps({"affine8": affine8_leg()}), flush=True)
        return
    if args.only == "stacked":
        print(json.dumps({"stacked": stacked_leg(min(args.steps, 20), min(args.warmup, 3))}), flush=True)
        return
    c = W.CONFIGS["decode"]
    log(f"building the bank: {c['E']} records of {wq.moe_nvfp4_record_bytes(c['H'], c['I'])} B")
    t0 = time.time()
    bank, base = W.build_bank(c["bank_seed"], c["H"], c["I"], c["E"])
    log(f"bank ready in {time.time() - t0:.1f} s")
    peaks = None if args.no_probes or args.only in ("cache", "verify", "batched") else probe_peaks(fast=True)
    if args.only == "prefill":
        print(json.dumps({"prefill": prefill_leg(bank, args.prefill_steps, peaks)}), flush=True)
        return
    if args.only == "cache":
        print(json.dumps({"expert_cache": cache_leg(bank, base)}), flush=True)
        return
    if args.only == "verify":
        print(json.dumps({"verify": verify_leg(bank, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "batched":
        print(json.dumps({"batched": batched_leg(bank, min(args.steps, 50), min(args.warmup, 5))}), flush=True)
        return

    # ---- decode leg
    dec = DecodeLeg(bank)
    dec.two_call = args.two_call
    K, Wm = args.steps, args.warmup
    ms_total, wall_ms = timed(dec.step, K, Wm)
    status = check_status(dec.ws, "decode")
    dec.idx_host = dec.idx.cpu().numpy()
    first = (Wm) % ROTATE
    rs = [(first + i) % ROTATE for i in range(K)]
    step_bytes = np.array([dec.step_bytes(r) for r in rs], dtype=np.float64)
    ms_per_step = ms_total / K
    value = step_bytes.sum() / (ms_total * 1e-3) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step, {value:.1f} GB/s (wall {wall_ms / K * 1e3:.1f} us/step)")

    dec.i = Wm
    dist = step_stats(dec.step, K)
    # per-kernel times from events around each launch (a separate pass: the
    # events add a little launch overhead)
    wq.moe_profile_enable(True)
    dec.i = Wm
    for _ in range(K):
        dec.step()
    torch.cuda.synchronize()
    kern = {}
    for name in ["router", "topk", "sort", "decode_route_gateup", "decode_gateup", "decode_down", "combine"]:
        avg, cnt = kernel_avg_ms(name)
        if cnt:
            kern[name] = (avg, cnt)
    wq.moe_profile_enable(False)
    for n_, (avg, cnt) in kern.items():
        log(f"  {n_:15s} {avg * 1e3:8.2f} us x {cnt}")
    gu_name = "decode_gateup" if dec.two_call else "decode_route_gateup"
    gu_bytes = np.mean([dec.gateup_bytes(r) for r in rs])
    gu_ms = kern[gu_name][0]
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    roofline = {"kernel": gu_name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(gu_name),
                "bytes_per_launch": int(gu_bytes), "avg_launch_us": round(gu_ms * 1e3, 2)}
    if peaks:
        pm = peaks["hbm_read_step_size_GBps"]
        roofline.update({"peak_measured": pm, "frac_measured": round(achieved / pm, 4),
                         "peak_measured_by": "streaming read of 182 MB pieces (moe_probe_hbm_read)"})

    out = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "decode: one NVFP4 MoE layer, T=1, H=5120, I=2560, 256 experts, top-8, "
                                  "router f32 5120x256; 64 rotating activations",
                      "global_batch": 1, "H": 5120, "I": 2560, "E": 256, "top_k": 8,
                      "bytes_per_step": int(step_bytes.mean())},
           "roofline": roofline, "step_us": dist, "status": status,
           "kernels_us": {n_: round(v[0] * 1e3, 2) for n_, v in kern.items()}}
    if peaks:
        out["peak_probes"] = peaks

    # ---- prefill leg
    if not args.no_prefill:
        del dec
        torch.cuda.empty_cache()
        out["prefill"] = prefill_leg(bank, args.prefill_steps, peaks)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
