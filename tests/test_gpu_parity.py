"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every oracle input comes from the seeded generators or from the oracle itself
(never from the HIP path). Comparison classes:
  bit-exact:  pack bytes, dequantized f32 weights and bf16 unit values, top-k
              indices on identical logits, the pair sort;
  bounded:    router logits (f32 sums in another order: 1e-5 rms), softmax
              weights (f32 evaluation, bound derived in check_weights), bf16
              outputs of the resident linear and the norm (one bf16 ulp +
              1e-4 rms, see check_bf16);
  rounding:   a bf16 layer output is the f32 output of the same inputs rounded
              once to nearest even, bit for bit (check_bf16_of); the f32
              output carries the tolerance below;
  tolerance:  f32 layer outputs, relative L2 <= 5e-3 and per-element
              |err| <= 1e-2 * rms(reference).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W

wq = pytest.importorskip("weight_quantized_moe_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def to_np_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_f32(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref**2))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.max(np.abs(got - ref)) / rms
    say(f"{what}: rel L2 {rel:.3e}, max |err|/rms {mx:.3e}")
    assert rel <= 5e-3 and mx <= 1e-2, (what, rel, mx)


def check_bf16(got_bits, ref_f32, what):
    """A bf16 output is the device's f32 value rounded once (half a bf16 ulp);
    the f32 value itself carries the f32 path's absolute error, which near a
    cancellation exceeds the bf16 ulp of the tiny result. Bound: one bf16 ulp of
    |ref| plus 1e-4 * rms(ref), a hundredth of the per-element layer bound."""
    got = oracle.bf16_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref_f32, np.float64)
    a = np.maximum(np.abs(ref), 2.0**-126)
    ulp = 2.0 ** (np.floor(np.log2(a)) - 7)
    rms = np.sqrt(np.mean(ref**2))
    err = np.abs(got - ref)
    bad = err > ulp + 1e-4 * rms
    say(f"{what}: max |err| - ulp = {np.max(err - ulp) / rms:.2e} rms")
    assert not bad.any(), (what, int(bad.sum()), got[bad][:5], ref[bad][:5])


def check_bf16_of(got_bits, got_f32, what):
    """The layer's bf16 output is its f32 result rounded once (RNE). The f32
    result is held to the layer tolerance by check_f32; near a cancellation its
    absolute error (f32 sums of a few thousand products, and bf16 mids that
    round differently from the float64 oracle's) exceeds a bf16 ulp of the
    small result, so the bf16 output is compared with the rounding of the f32
    output, which must match exactly."""
    want = oracle.f64_to_bf16(np.asarray(got_f32, np.float64))
    got = np.asarray(got_bits, np.uint16)
    bad = got != want
    say(f"{what}: bf16 == rne(f32) on {got.size - int(bad.sum())}/{got.size}")
    assert not bad.any(), (what, int(bad.sum()), got[bad][:5], want[bad][:5])


def host_records(seed, experts, H, I):
    recs = {}
    for e in experts:
        c, s, g = W.host_parts(seed, int(e), H, I)
        recs[int(e)] = oracle.pack_record(H, I, c, s, g)
    return recs


def oracle_routing(name, x, Wr, logits, k):
    if logits is None:
        logits = oracle.router_logits(x, Wr)
    idx, w = oracle.route_topk(logits, k)
    return logits, idx, w


def gpu_forward(bank, x_bits, idx, w, k, flags=0, residual=None):
    T, H = x_bits.shape
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, bank.H, bank.I, bank.E))
    xd = bf16_tensor(x_bits)
    idd = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV)
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV)
    rd = None if residual is None else bf16_tensor(residual)
    yf = torch.empty((T, H), dtype=torch.float32, device=DEV)
    yb = torch.empty((T, H), dtype=torch.int16, device=DEV)
    wq.moe_nvfp4_forward(bank, xd, T, idd, wd, k, rd, yf, flags | wq.MOE_F32_OUT, ws)
    wq.moe_nvfp4_forward(bank, xd, T, idd, wd, k, rd, yb, flags, ws)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), to_np_bits(yb)


# ---- banks ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny_bank():
    c = W.CONFIGS["tiny"]
    say("building tiny bank")
    return W.build_bank(c["bank_seed"], c["H"], c["I"], c["E"])


@pytest.fixture(scope="module")
def big_bank():
    c = W.CONFIGS["decode"]
    say("building the 256-record bank (5.66 GB)")
    return W.build_bank(c["bank_seed"], c["H"], c["I"], c["E"])


# ---- S0 pack and the dequant rule --------------------------------------------------
def test_pack_bytes_match_oracle_tiny(tiny_bank):
    bank, base = tiny_bank
    c = W.CONFIGS["tiny"]
    recs = host_records(c["bank_seed"], range(c["E"]), c["H"], c["I"])
    dev = base.cpu().numpy()
    for e in range(c["E"]):
        assert np.array_equal(dev[e * bank.stride:(e + 1) * bank.stride], recs[e]), e


def test_pack_bytes_match_oracle_sampled_full_shape(big_bank):
    bank, base = big_bank
    c = W.CONFIGS["decode"]
    for e in [0, 1, 97, 255]:
        rec = host_records(c["bank_seed"], [e], c["H"], c["I"])[e]
        dev = base[e * bank.stride:(e + 1) * bank.stride].cpu().numpy()
        assert np.array_equal(dev, rec), e


# ---- 8-dim VQ experts -------------------------------------------------------------------
def vq_host_records(seed, experts, H, I):
    recs = {}
    for e in experts:
        idx, gains = synth.vq_expert_parts(seed, int(e), H, I)
        recs[int(e)] = oracle.vq_pack_record(H, I, [a.numpy() for a in idx], gains)
    return recs


@pytest.fixture(scope="module")
def vq_tiny():
    say("building the tiny VQ bank")
    return W.build_vq_bank(31, 256, 128, 16)


@pytest.fixture(scope="module")
def vq_big():
    say("building the 256-record VQ bank (1.89 GB)")
    return W.build_vq_bank(32, 5120, 2560, 256)


def test_vq_pack_and_dequant_bit_exact(vq_tiny, vq_big):
    for (bank, base, cb), H, I, seed, experts in [(vq_tiny, 256, 128, 31, range(16)), (vq_big, 5120, 2560, 32, [0, 201])]:
        recs = vq_host_records(seed, experts, H, I)
        cbh = cb.cpu().numpy()
        for e in experts:
            assert np.array_equal(base[e * bank.stride:(e + 1) * bank.stride].cpu().numpy(), recs[e]), e
            for p in range(3):
                out, inn = oracle.proj_shape(H, I, p)
                d = torch.empty((out, inn), dtype=torch.float32, device=DEV)
                wq.moe_vq_dequant(bank, e, p, d)
                torch.cuda.synchronize()
                ref = oracle.vq_dequant_projection(recs[e], cbh, H, I, p)
                assert np.array_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, p)


def gpu_vq_forward(bank, x_bits, idx, w, k, residual=None):
    T, H = x_bits.shape
    ws = wq.workspace(wq.moe_vq_workspace_bytes(T, k, bank.H, bank.I))
    xd = bf16_tensor(x_bits)
    idd = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV)
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV)
    rd = None if residual is None else bf16_tensor(residual)
    yf = torch.empty((T, H), dtype=torch.float32, device=DEV)
    yb = torch.empty((T, H), dtype=torch.int16, device=DEV)
    wq.moe_vq_forward(bank, xd, T, idd, wd, k, rd, yf, wq.MOE_F32_OUT, ws)
    wq.moe_vq_forward(bank, xd, T, idd, wd, k, rd, yb, 0, ws)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), to_np_bits(yb)


def test_vq_forward_tiny(vq_tiny):
    bank, base, cb = vq_tiny
    H, I, E, k, T = 256, 128, 16, 2, 5
    x = synth.activations(33, T, H)
    lg = np.random.default_rng(33).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    res = synth.activations(34, T, H)
    recs = vq_host_records(31, np.unique(idx), H, I)
    for residual in (None, res):
        yf, yb = gpu_vq_forward(bank, x, idx, w, k, residual)
        rf, _ = oracle.vq_moe_forward(recs, cb.cpu().numpy(), E, H, I, x, idx, w, residual=residual)
        check_f32(yf, rf, "vq tiny")
        check_bf16_of(yb, yf, "vq tiny bf16")


@pytest.mark.parametrize("T", [1, 3])
def test_vq_forward_full_shape(vq_big, T):
    # T = 1: single-token decode; T = 3: a short verify pass of a few tokens
    bank, base, cb = vq_big
    H, I, E, k = 5120, 2560, 256, 8
    x = synth.activations(35 + T, T, H)
    _, Wr, _ = W.inputs("decode")
    lg = oracle.router_logits(x, Wr)
    idx, w = oracle.route_topk(lg, k)
    recs = vq_host_records(32, np.unique(idx), H, I)
    yf, yb = gpu_vq_forward(bank, x, idx, w, k)
    rf, _ = oracle.vq_moe_forward(recs, cb.cpu().numpy(), E, H, I, x, idx, w)
    check_f32(yf, rf, f"vq T={T}")
    check_bf16_of(yb, yf, f"vq T={T} bf16")


def test_vq_forward_odd_k_two_passes_dropped_slot():
    # k = 3: the gate/up workgroups take slots in twos, the last alone; H and
    # I one group past a lane's five (81 and 41 groups): a second pass over
    # each row; a slot with id -1 contributes nothing (the oracle gets a valid
    # id with routing weight 0 there)
    H, I, E, k, T = 5184, 2624, 6, 3, 4
    say(f"vq H={H} I={I} k={k}")
    bank, base, cb = W.build_vq_bank(37, H, I, E)
    x = synth.activations(38, T, H)
    lg = np.random.default_rng(38).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    recs = vq_host_records(37, np.unique(idx), H, I)
    res = synth.activations(39, T, H)
    idx_gpu = idx.copy()
    idx_gpu[1, 2] = -1
    w_ref = w.copy()
    w_ref[1, 2] = 0.0
    yf, yb = gpu_vq_forward(bank, x, idx_gpu, w, k, res)
    rf, _ = oracle.vq_moe_forward(recs, cb.cpu().numpy(), E, H, I, x, idx, w_ref, residual=res)
    check_f32(yf, rf, "vq odd k")
    check_bf16_of(yb, yf, "vq odd k bf16")


# ---- pack side: record digests and the manifest --------------------------------------
def device_digests(bank, e0, n):
    d = torch.empty((n, 32), dtype=torch.uint8, device=DEV)
    wq.moe_nvfp4_record_sha256(bank, e0, n, d)
    torch.cuda.synchronize()
    return [bytes(r) for r in d.cpu().numpy()]


@pytest.mark.parametrize("H,I,E", [(256, 128, 16), (16, 16, 5), (16, 32, 3)])
def test_record_sha256_small_banks(H, I, E):
    # record sizes end 12, 60 and 44 bytes into a 64-byte block: one and two
    # padding blocks
    import hashlib
    seed = 11
    say(f"sha256 of {E} records at H={H} I={I}")
    bank, base = W.build_bank(seed, H, I, E)
    _, nbytes, _ = oracle.record_layout(H, I)
    recs = host_records(seed, range(E), H, I)
    want = [hashlib.sha256(recs[e][:nbytes].tobytes()).digest() for e in range(E)]
    assert device_digests(bank, 0, E) == want
    assert device_digests(bank, 1, E - 2) == want[1:E - 1]


def test_record_sha256_full_shape_sampled(big_bank):
    import hashlib
    bank, base = big_bank
    c = W.CONFIGS["decode"]
    _, nbytes, _ = oracle.record_layout(c["H"], c["I"])
    got = device_digests(bank, 96, 2) + device_digests(bank, 255, 1)
    recs = host_records(c["bank_seed"], [96, 97, 255], c["H"], c["I"])
    want = [hashlib.sha256(recs[e][:nbytes].tobytes()).digest() for e in (96, 97, 255)]
    assert got == want


def test_manifest_with_recovered_global_scales():
    # the pack-side flow: weight_scale_2 values -> g (library, host) -> records
    # holding those g -> manifest; the oracle repacks the same parts with the
    # oracle's own g and hashes them
    import hashlib
    from weight_quantized_moe_amd import manifest
    H, I, E, seed = 256, 128, 8, 12
    bank, base = W.build_bank(seed, H, I, E)
    rng = np.random.default_rng(7)
    ws2 = np.exp(rng.uniform(np.log(1e-4), np.log(1e-1), (E, 3))).astype(np.float32)
    g, inexact = wq.moe_nvfp4_global_from_ws2(ws2.ravel())
    g_ref, inexact_ref = oracle.global_from_ws2(ws2.ravel())
    assert np.array_equal(g.view(np.uint32), g_ref.view(np.uint32)) and np.array_equal(inexact, inexact_ref)
    g, inexact = g.reshape(E, 3), inexact.reshape(E, 3)
    for e in range(E):
        for p in range(3):
            off = e * bank.stride + int(bank.part_off[6 + p])
            base[off:off + 4] = torch.from_numpy(g[e, p:p + 1].view(np.uint8).copy()).to(DEV)
    torch.cuda.synchronize()
    m = manifest.bank_manifest(bank, inexact)
    _, nbytes, stride = oracle.record_layout(H, I)
    want_inexact = [(e, manifest.PROJECTIONS[p]) for e in range(E) for p in range(3) if inexact_ref[e * 3 + p]]
    assert [(r["record"], r["projection"]) for r in m["global_scale_inexact"]] == want_inexact
    for e in range(E):
        c_, s_, _ = W.host_parts(seed, e, H, I)
        rec = oracle.pack_record(H, I, c_, s_, g_ref[3 * e:3 * e + 3])
        assert m["records"][e] == {"offset": e * stride, "length": nbytes,
                                   "sha256": hashlib.sha256(rec[:nbytes].tobytes()).hexdigest()}, e


# ---- expert cache: records in HBM slots, fed from pinned host memory ------------------
def run_through_cache(dev_bank, dev_base, nslots, steps):
    """steps: [(x_bits [T][H], idx [T][k], w [T][k])]. Each step prepares the
    step's distinct experts (first-appearance order) in a cache over a pinned
    host copy of the bank, runs the forward on the slot pool with idx mapped to
    slots, and the same forward on the full device bank. Returns the outputs of
    both, the slots and the per-step counts."""
    host_mem = torch.empty(dev_base.numel(), dtype=torch.uint8, pin_memory=True)
    host_mem.copy_(dev_base)
    host_bank = wq.moe_nvfp4_bank()
    host_bank.H, host_bank.I, host_bank.E = dev_bank.H, dev_bank.I, dev_bank.E
    host_bank.record_bytes, host_bank.stride = dev_bank.record_bytes, dev_bank.stride
    for i in range(9):
        host_bank.part_off[i] = dev_bank.part_off[i]
    host_bank.base = host_mem.data_ptr()
    slots_mem = torch.empty(nslots * dev_bank.stride + 4096, dtype=torch.uint8, device=DEV)
    off = (-slots_mem.data_ptr()) % 4096
    slot_base = slots_mem[off:off + nslots * dev_bank.stride]
    cache = wq.moe_cache_create(host_bank, slot_base, nslots)
    try:
        cb = wq.moe_cache_bank(cache)
        cache_out, full_out, slots, counts = [], [], [], []
        for x, idx, w in steps:
            ids = list(dict.fromkeys(int(e) for e in np.asarray(idx).ravel()))
            h0, m0, _ = wq.moe_cache_stats(cache)
            slot_of = wq.moe_cache_prepare(cache, ids)
            h1, m1, _ = wq.moe_cache_stats(cache)
            remap = dict(zip(ids, slot_of.tolist()))
            sidx = np.vectorize(remap.get)(np.asarray(idx)).astype(np.int32)
            k = idx.shape[1]
            cache_out.append(gpu_forward(cb, x, sidx, w, k))
            full_out.append(gpu_forward(dev_bank, x, idx, w, k))
            slots.append(slot_of.tolist())
            counts.append((h1 - h0, m1 - m0))
        return cache_out, full_out, slots, counts, wq.moe_cache_stats(cache)
    finally:
        wq.moe_cache_destroy(cache)


def check_cache_run(nslots, steps, result, stride):
    cache_out, full_out, slots, counts, (hits, misses, nbytes) = result
    calls = [list(dict.fromkeys(int(e) for e in np.asarray(idx).ravel())) for _, idx, _ in steps]
    want = oracle.lru_slots(nslots, calls)
    for t in range(len(steps)):
        assert slots[t] == want[t][0], t
        assert counts[t] == (want[t][1], want[t][2]), t
        # the same kernels on the same record bytes: identical outputs
        assert np.array_equal(cache_out[t][0].view(np.uint32), full_out[t][0].view(np.uint32)), t
        assert np.array_equal(cache_out[t][1], full_out[t][1]), t
    assert misses == sum(m for _, _, m in want) and hits == sum(h for _, h, _ in want)
    assert nbytes == misses * stride
    say(f"cache of {nslots}: {hits} hits, {misses} misses over {len(steps)} steps")


def test_expert_cache_tiny(tiny_bank):
    bank, base = tiny_bank
    c = W.CONFIGS["tiny"]
    rng = np.random.default_rng(21)
    x, _, _ = W.inputs("tiny")
    steps = []
    for t in range(40):
        idx = np.stack([rng.choice(c["E"], size=c["k"], replace=False) for _ in range(2)]).astype(np.int32)
        w = rng.uniform(0.1, 1.0, idx.shape).astype(np.float32)
        steps.append((x[:2], idx, w))
    check_cache_run(5, steps, run_through_cache(bank, base, 5, steps), bank.stride)


def test_expert_cache_decode_full_shape(big_bank):
    # single-token decode steps with Zipf-skewed routing (the batched config's
    # 32 tokens, one per step), 64 slots of 256
    bank, base = big_bank
    c = W.CONFIGS["batched"]
    x, _, logits = W.inputs("batched")
    idx, w = oracle.route_topk(logits, c["k"])
    steps = [(x[t:t + 1], idx[t:t + 1], w[t:t + 1]) for t in range(16)]
    check_cache_run(64, steps, run_through_cache(bank, base, 64, steps), bank.stride)


@pytest.mark.parametrize("proj", [0, 1, 2])
def test_dequant_bit_exact_tiny(tiny_bank, proj):
    bank, base = tiny_bank
    c = W.CONFIGS["tiny"]
    rows, cols = (c["H"], c["I"]) if proj == 2 else (c["I"], c["H"])
    recs = host_records(c["bank_seed"], range(c["E"]), c["H"], c["I"])
    for e in range(c["E"]):
        wf = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
        wu = torch.empty((rows, cols), dtype=torch.int16, device=DEV)
        wq.moe_nvfp4_dequant(bank, e, proj, wf, wu)
        torch.cuda.synchronize()
        rw, ru = oracle.dequant_projection(recs[e], c["H"], c["I"], proj)
        assert np.array_equal(wf.cpu().numpy().view(np.uint32), rw.view(np.uint32)), (e, proj)
        assert np.array_equal(to_np_bits(wu), ru), (e, proj)


def test_dequant_bit_exact_full_shape(big_bank):
    bank, base = big_bank
    c = W.CONFIGS["decode"]
    for e, proj in [(3, 0), (128, 1), (254, 2)]:
        rows, cols = (c["H"], c["I"]) if proj == 2 else (c["I"], c["H"])
        rec = host_records(c["bank_seed"], [e], c["H"], c["I"])[e]
        wf = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
        wu = torch.empty((rows, cols), dtype=torch.int16, device=DEV)
        wq.moe_nvfp4_dequant(bank, e, proj, wf, wu)
        torch.cuda.synchronize()
        rw, ru = oracle.dequant_projection(rec, c["H"], c["I"], proj)
        assert np.array_equal(wf.cpu().numpy().view(np.uint32), rw.view(np.uint32)), (e, proj)
        assert np.array_equal(to_np_bits(wu), ru), (e, proj)


# ---- S1 + S2 routing -----------------------------------------------------------------
def gpu_route(x_bits, Wr, logits_in, E, k):
    T, H = x_bits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    if logits_in is None:
        lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
        wq.moe_route_topk(bf16_tensor(x_bits), torch.from_numpy(Wr).to(DEV), lg, T, H, E, k, idx, w)
    else:
        lg = torch.from_numpy(np.ascontiguousarray(logits_in)).to(DEV)
        wq.moe_route_topk(None, None, lg, T, H, E, k, idx, w)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check_weights(w_gpu, w_ref, logits_sel):
    """Softmax weights: the device evaluates w_j = expf(l_j - l_0) / sum in f32.
    With unit roundoff u = 2^-24: the difference costs |l_j - l_0| u, expf
    about 2u, the k-term sum (k - 1)u, the division u, relative to w_j. The
    bound doubles that: (|l_j - l_0| + k + 3) * 2u * w_j."""
    k = w_ref.shape[1]
    d = np.abs(logits_sel.astype(np.float64) - logits_sel[:, :1].astype(np.float64))
    tol = (d + k + 3) * 2.0**-23 * np.abs(w_ref.astype(np.float64))
    err = np.abs(w_gpu.astype(np.float64) - w_ref.astype(np.float64))
    assert np.all(err <= tol), float(np.max(err / np.maximum(tol, 1e-300)))


@pytest.mark.parametrize("name", ["tiny", "decode", "stacked"])
def test_router_logits_and_topk(name):
    c = W.CONFIGS[name]
    for variant in range(3):
        x, Wr, _ = W.inputs(name, variant)
        ref_lg = oracle.router_logits(x, Wr)
        lg, _, _ = gpu_route(x, Wr, None, c["E"], c["k"])
        rms = np.sqrt(np.mean(ref_lg.astype(np.float64) ** 2))
        assert np.max(np.abs(lg - ref_lg)) <= 1e-5 * rms, name
        # top-k on identical logits (the oracle's): bit-exact indices
        _, idx, w = gpu_route(x, None, ref_lg, c["E"], c["k"])
        ridx, rw = oracle.route_topk(ref_lg, c["k"])
        assert np.array_equal(idx, ridx)
        check_weights(w, rw, np.take_along_axis(ref_lg, ridx, axis=1))


@pytest.mark.parametrize("name", ["batched", "prefill"])
def test_topk_on_given_logits(name):
    c = W.CONFIGS[name]
    x, _, logits = W.inputs(name)
    _, idx, w = gpu_route(x, None, logits, c["E"], c["k"])
    ridx, rw = oracle.route_topk(logits, c["k"])
    assert np.array_equal(idx, ridx)
    check_weights(w, rw, np.take_along_axis(logits, ridx, axis=1))


def test_topk_ties_zeros_and_k_edges():
    rng = np.random.default_rng(0)
    for E, k in [(256, 8), (1024, 64), (16, 16), (5, 1), (64, 3)]:
        lg = rng.normal(size=(37, E)).astype(np.float32)
        lg[0] = 0.0
        lg[1, ::2] = -0.0
        lg[2] = np.round(lg[2])
        lg[3, :] = 7.0
        x = np.zeros((37, 16), np.uint16)
        _, idx, w = gpu_route(x, None, lg, E, k)
        ridx, rw = oracle.route_topk(lg, k)
        assert np.array_equal(idx, ridx), (E, k)
        check_weights(w, rw, np.take_along_axis(lg, ridx, axis=1))


# ---- S3 sort -------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (32, 8, 256), (8192, 8, 256), (4, 2, 16), (3, 64, 1024), (1, 1, 1)])
def test_sort_bit_exact(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    srt = torch.empty(T * k, dtype=torch.int32, device=DEV)
    wq.moe_sort_pairs(torch.from_numpy(idx).to(DEV), T, k, E, offs, srt)
    torch.cuda.synchronize()
    roff, rsrt = oracle.sort_pairs(idx, E)
    assert np.array_equal(offs.cpu().numpy(), roff)
    assert np.array_equal(srt.cpu().numpy(), rsrt)


@pytest.mark.parametrize("T,k,E", [(8192, 8, 256), (300, 8, 256), (257, 8, 16), (5000, 3, 1024), (2000, 64, 1000)])
def test_sort_multi_workgroup_bit_exact(T, k, E):
    """moe_sort_pairs_ws: above 2048 pairs the count / scan / place launches;
    the same stable order and offsets as the oracle (ragged last chunks, E up
    to 1024, a Zipf-skewed case with large groups)."""
    rng = np.random.default_rng(T * 13 + k)
    if T == 8192:
        _, _, logits = W.inputs("prefill")
        idx, _ = oracle.route_topk(logits, k)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[0, 0] = -1 if T == 5000 else idx[0, 0]  # one dropped pair
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    srt = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(wq.moe_sort_workspace_bytes(T, k, E) // 4 + 1, dtype=torch.int32, device=DEV)
    wq.moe_sort_pairs_ws(torch.from_numpy(idx).to(DEV), T, k, E, offs, srt, ws)
    torch.cuda.synchronize()
    flat = idx.ravel()
    keep = np.nonzero((flat >= 0) & (flat < E))[0]  # the oracle takes valid pairs only
    roff, rsrt = oracle.sort_pairs(flat[keep], E)
    assert np.array_equal(offs.cpu().numpy(), roff)
    n = int(roff[-1])
    assert n == keep.size
    assert np.array_equal(srt.cpu().numpy()[:n], keep[rsrt])


def test_sort_drops_invalid_indices():
    idx = np.array([[3, -1], [7, 3], [16, 0]], np.int32)
    offs = torch.empty(17, dtype=torch.int32, device=DEV)
    srt = torch.full((6,), -5, dtype=torch.int32, device=DEV)
    wq.moe_sort_pairs(torch.from_numpy(idx).to(DEV), 3, 2, 16, offs, srt)
    torch.cuda.synchronize()
    valid = idx.ravel()[(idx.ravel() >= 0) & (idx.ravel() < 16)]
    roff, _ = oracle.sort_pairs(valid, 16)
    assert np.array_equal(offs.cpu().numpy(), roff)
    assert srt.cpu().numpy()[:4].tolist() == [5, 0, 3, 2]


# ---- the layer -------------------------------------------------------------------------
@pytest.mark.parametrize("flags", [0, 2, 4])  # auto, forced GEMV, forced grouped GEMM
def test_forward_tiny(tiny_bank, flags):
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    recs = host_records(c["bank_seed"], range(c["E"]), c["H"], c["I"])
    for variant in range(3):
        x, Wr, _ = W.inputs("tiny", variant)
        _, idx, w = oracle_routing("tiny", x, Wr, None, c["k"])
        ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w)
        yf, yb = gpu_forward(bank, x, idx, w, c["k"], flags)
        check_f32(yf, ref_f, f"tiny flags={flags} v{variant}")
        check_bf16_of(yb, yf, "tiny bf16")


def test_forward_tiny_ragged_and_residual(tiny_bank):
    # T not a multiple of any tile, duplicated experts across tokens, an
    # expert with many tokens (grouped-GEMM tail), a residual input
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    recs = host_records(c["bank_seed"], range(c["E"]), c["H"], c["I"])
    T, k = 203, 2
    x = synth.activations(77, T, c["H"])
    res = synth.activations(78, T, c["H"])
    lg = np.random.default_rng(5).normal(size=(T, c["E"])).astype(np.float32)
    lg[:, 3] += 3.0  # expert 3 in nearly every token
    idx, w = oracle.route_topk(lg, k)
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w, residual=res)
    for flags in (2, 4):
        yf, yb = gpu_forward(bank, x, idx, w, k, flags, residual=res)
        check_f32(yf, ref_f, f"tiny ragged flags={flags}")
        check_bf16_of(yb, yf, "tiny ragged bf16")


def test_forward_partial_output_tiles():
    # H = 320, I = 192: the grouped GEMM's last n-tile is partial in both
    # launches (gate/up 128 output columns a tile, down 256), so the
    # epilogues' column masks and their row-piece stores meet a tile edge;
    # K of 5 and 3 k-steps (odd) and ragged row tiles
    H, I, E, T, k = 320, 192, 8, 150, 2
    say(f"partial output tiles H={H} I={I} E={E} T={T}")
    bank, _ = W.build_bank(3, H, I, E)
    recs = host_records(3, range(E), H, I)
    x = synth.activations(91, T, H)
    res = synth.activations(92, T, H)
    lg = np.random.default_rng(9).normal(size=(T, E)).astype(np.float32)
    lg[:, 5] += 2.0
    idx, w = oracle.route_topk(lg, k)
    ref_f, _ = oracle.moe_forward(recs, E, H, I, x, idx, w, residual=res)
    for flags in (2, 4):
        yf, yb = gpu_forward(bank, x, idx, w, k, flags, residual=res)
        check_f32(yf, ref_f, f"partial tiles flags={flags}")
        check_bf16_of(yb, yf, "partial tiles bf16")


def test_forward_single_token_paths(tiny_bank):
    # one token takes the flat kernels (k <= 16); k = 16 is their largest case,
    # the residual is folded into their combine; flags=2 forces the same path
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    recs = host_records(c["bank_seed"], range(c["E"]), c["H"], c["I"])
    for k, seed in [(2, 31), (1, 32), (16, 33), (7, 34)]:
        x = synth.activations(seed, 1, c["H"])
        res = synth.activations(seed + 100, 1, c["H"])
        lg = np.random.default_rng(seed).normal(size=(1, c["E"])).astype(np.float32)
        idx, w = oracle.route_topk(lg, k)
        for residual in (None, res):
            ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w, residual=residual)
            for flags in (0, 4):
                yf, yb = gpu_forward(bank, x, idx, w, k, flags, residual=residual)
                check_f32(yf, ref_f, f"one token k={k} flags={flags} residual={residual is not None}")
                check_bf16_of(yb, yf, "one token bf16")


def test_forward_decode_full_shape(big_bank):
    bank, _ = big_bank
    c = W.CONFIGS["decode"]
    for variant in range(2):
        x, Wr, _ = W.inputs("decode", variant)
        _, idx, w = oracle_routing("decode", x, Wr, None, c["k"])
        say(f"decode v{variant}: experts {idx.ravel().tolist()}")
        recs = host_records(c["bank_seed"], np.unique(idx), c["H"], c["I"])
        ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w)
        for flags in (0, 4):
            yf, yb = gpu_forward(bank, x, idx, w, c["k"], flags)
            check_f32(yf, ref_f, f"decode v{variant} flags={flags}")
            check_bf16_of(yb, yf, "decode bf16")


@pytest.mark.parametrize("T", [2, 4])
def test_forward_verify_shape_full(big_bank, T):
    # a draft-verify pass of a few tokens (the multi-token expert-streaming
    # path, routed inside its blocks), with a residual, against the oracle;
    # and the one-call layer against route + forward
    bank, _ = big_bank
    c = W.CONFIGS["decode"]
    x = synth.activations(40 + T, T, c["H"])
    res = synth.activations(50 + T, T, c["H"])
    _, Wr, _ = W.inputs("decode")
    _, idx, w = oracle_routing("decode", x, Wr, None, c["k"])
    say(f"verify T={T}: {len(np.unique(idx))} distinct experts")
    recs = host_records(c["bank_seed"], np.unique(idx), c["H"], c["I"])
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w, residual=res)
    yf, yb = gpu_forward(bank, x, idx, w, c["k"], 0, res)
    check_f32(yf, ref_f, f"verify T={T}")
    check_bf16_of(yb, yf, f"verify T={T} bf16")
    check_layer_call(bank, f"verify T={T}", x, Wr, c["k"], residual=res)


def gpu_layer(bank, x_bits, Wr, k, flags=0, residual=None, ws=None):
    """moe_nvfp4_layer: router, top-k and layer in one call. Returns logits,
    idx, w, y f32 and y bf16 (two calls, the second with the f32 flag off) and
    the workspace's status word."""
    T, H = x_bits.shape
    E = Wr.shape[0]
    if ws is None:
        ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, bank.H, bank.I, bank.E))
    wq.moe_status_clear(ws)  # the status word: set only if a bounded wait expires
    xd = bf16_tensor(x_bits)
    wrd = torch.from_numpy(np.ascontiguousarray(Wr)).to(DEV)
    rd = None if residual is None else bf16_tensor(residual)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    yf = torch.empty((T, H), dtype=torch.float32, device=DEV)
    yb = torch.empty((T, H), dtype=torch.int16, device=DEV)
    wq.moe_nvfp4_layer(bank, xd, wrd, T, k, rd, lg, idx, w, yf, flags | wq.MOE_F32_OUT, ws)
    wq.moe_nvfp4_layer(bank, xd, wrd, T, k, rd, lg, idx, w, yb, flags, ws)
    torch.cuda.synchronize()
    status = wq.moe_status_read(ws)
    return lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), yf.cpu().numpy(), to_np_bits(yb), status


def check_layer_call(bank, name, x, Wr, k, residual=None, ws=None, flags=0):
    """The one-call layer against the two-call path it stands for (router and
    top-k by moe_route_topk, then moe_nvfp4_forward on its idx and w): logits,
    idx, w and both outputs bit for bit; the separate path is held to the
    oracle by the tests above and here again through the logits."""
    lg, idx, w, yf, yb, status = gpu_layer(bank, x, Wr, k, flags, residual, ws)
    assert status == 0, (name, status)
    lg2, idx2, w2 = gpu_route(x, Wr, None, bank.E, k)
    assert np.array_equal(lg.view(np.uint32), lg2.view(np.uint32)), (name, "logits")
    assert np.array_equal(idx, idx2), (name, "idx")
    assert np.array_equal(w.view(np.uint32), w2.view(np.uint32)), (name, "w")
    yf2, yb2 = gpu_forward(bank, x, idx2, w2, k, flags, residual)
    assert np.array_equal(yf.view(np.uint32), yf2.view(np.uint32)), (name, "y f32")
    assert np.array_equal(yb, yb2), (name, "y bf16")
    ref_lg = oracle.router_logits(x, Wr)
    rms = np.sqrt(np.mean(ref_lg.astype(np.float64) ** 2))
    assert np.max(np.abs(lg - ref_lg)) <= 1e-5 * rms, (name, "logits vs oracle")
    say(f"layer call {name}: matches route + forward bit for bit")
    return idx, w, yf


def test_layer_call_tiny(tiny_bank):
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    x, Wr, _ = W.inputs("tiny")
    check_layer_call(bank, "tiny T=4", x, Wr, c["k"])
    check_layer_call(bank, "tiny T=4 grouped GEMM", x, Wr, c["k"], flags=4)
    res = synth.activations(77, c["T"], c["H"])
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(1, 8, bank.H, bank.I, bank.E))
    for t in range(c["T"]):  # one token: router and top-k inside the gate/up launch
        for kk in (1, 2, 8, 16):
            check_layer_call(bank, f"tiny token {t} k={kk}", x[t:t + 1], Wr, kk, res[t:t + 1] if t % 2 else None,
                             ws if kk <= 8 else None)


def test_many_experts_all_paths():
    # E = 600 (above 512: the one-token selection holds 16 keys per lane;
    # not a power of two), H = 128, I = 64, k = 4: the one-call layer on one
    # token against route + forward, and the forward through each path
    # (few-token kernels, routed GEMV, grouped GEMM) against the oracle
    H, I, E, k = 128, 64, 600, 4
    say(f"many experts: E={E}")
    bank, _ = W.build_bank(5, H, I, E)
    Wr = synth.router_weights(6, H, E)
    x1 = synth.activations(61, 1, H)
    idx1, _, _ = check_layer_call(bank, "E=600 one token", x1, Wr, k)
    assert np.all((idx1 >= 0) & (idx1 < E))
    for T, flags in ((4, 0), (40, 0), (300, 0), (300, 2)):
        x = synth.activations(62 + T, T, H)
        lg = np.random.default_rng(T).normal(size=(T, E)).astype(np.float32)
        lg[:, 17] += 2.5  # one expert in most tokens: a long group
        idx, w = oracle.route_topk(lg, k)
        recs = host_records(5, np.unique(idx), H, I)
        ref_f, _ = oracle.moe_forward(recs, E, H, I, x, idx, w)
        yf, yb = gpu_forward(bank, x, idx, w, k, flags)
        check_f32(yf, ref_f, f"E={E} T={T} flags={flags}")
        check_bf16_of(yb, yf, f"E={E} T={T} bf16")


def test_layer_call_decode_full_shape(big_bank):
    bank, _ = big_bank
    c = W.CONFIGS["decode"]
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(1, c["k"], c["H"], c["I"], c["E"]))
    for variant in range(3):  # one workspace: the tags of earlier calls stay behind
        x, Wr, _ = W.inputs("decode", variant)
        idx, w, yf = check_layer_call(bank, f"decode v{variant}", x, Wr, c["k"], ws=ws)
        ridx, rw = oracle.route_topk(oracle.router_logits(x, Wr), c["k"])
        assert np.array_equal(idx, ridx)
        recs = host_records(c["bank_seed"], np.unique(idx), c["H"], c["I"])
        ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, ridx, rw)
        check_f32(yf, ref_f, f"layer call decode v{variant}")


def test_forward_batched_full_shape(big_bank):
    # the batched-decode workload, every one of its 32 tokens against the oracle
    bank, _ = big_bank
    c = W.CONFIGS["batched"]
    x, _, logits = W.inputs("batched")
    idx, w = oracle.route_topk(logits, c["k"])
    yf, yb = gpu_forward(bank, x, idx, w, c["k"])
    recs = host_records(c["bank_seed"], np.unique(idx), c["H"], c["I"])
    say(f"batched: {len(recs)} distinct experts, all {c['T']} tokens")
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x, idx, w)
    check_f32(yf, ref_f, "batched T=32")
    check_bf16_of(yb, yf, "batched bf16")


def test_forward_routed_gemv_full_shape(big_bank):
    # 48 tokens on skewed logits: past the one-item-per-wave path, below the
    # grouped GEMM, i.e. the routed GEMV (sorted pairs, shared experts read
    # once); sampled tokens against the oracle
    bank, _ = big_bank
    c = W.CONFIGS["batched"]
    T = 48
    x = synth.activations(60, T, c["H"])
    logits = synth.skewed_logits(61, T, c["E"], rank_seed=c["seed"])
    idx, w = oracle.route_topk(logits, c["k"])
    res = synth.activations(62, T, c["H"])
    yf, yb = gpu_forward(bank, x, idx, w, c["k"], 0, res)
    sample = np.array([0, 1, 17, 30, 47])
    recs = host_records(c["bank_seed"], np.unique(idx[sample]), c["H"], c["I"])
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x[sample], idx[sample], w[sample], residual=res[sample])
    check_f32(yf[sample], ref_f, "routed gemv T=48 sampled")
    check_bf16_of(yb[sample], yf[sample], "routed gemv bf16")


@pytest.mark.parametrize("T", [9, 10, 14])
def test_flat_and_gemv_paths_at_the_token_limit(T, big_bank, monkeypatch):
    # up to 9 tokens take the one-item-per-wave kernels, from 10 the routed
    # GEMV; at the limit both paths (forced with MOE_FLAT_MAX_T) and the
    # default one must each match the oracle on sampled tokens
    bank, _ = big_bank
    c = W.CONFIGS["batched"]
    x = synth.activations(400 + T, T, c["H"])
    lg = synth.skewed_logits(410 + T, T, c["E"], rank_seed=c["seed"])
    idx, w = oracle.route_topk(lg, c["k"])
    res = synth.activations(420 + T, T, c["H"])
    sample = np.array([0, T // 2, T - 1])
    recs = host_records(c["bank_seed"], np.unique(idx[sample]), c["H"], c["I"])
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x[sample], idx[sample], w[sample],
                                  residual=res[sample])
    for lim in [None, "64", "1"]:
        if lim is None:
            monkeypatch.delenv("MOE_FLAT_MAX_T", raising=False)
        else:
            monkeypatch.setenv("MOE_FLAT_MAX_T", lim)
        yf, yb = gpu_forward(bank, x, idx, w, c["k"], 0, res)
        check_f32(yf[sample], ref_f, f"T={T} flat limit {lim or 'default'}")
        check_bf16_of(yb[sample], yf[sample], f"T={T} flat limit {lim or 'default'} bf16")
    monkeypatch.delenv("MOE_FLAT_MAX_T", raising=False)


def test_routed_gemv_inblock_routing_matches_tables(big_bank, monkeypatch):
    # 24 tokens take the routed GEMV; its blocks read their expert and pairs
    # from the sort tables, or (MOE_GEMV_INBLOCK=1, up to 256 pairs) find them
    # in idx themselves: same pairs in the same order, so bit-identical
    bank, _ = big_bank
    c = W.CONFIGS["batched"]
    T = 24
    x = synth.activations(91, T, c["H"])
    lg = synth.skewed_logits(92, T, c["E"], rank_seed=93)
    idx, w = oracle.route_topk(lg, c["k"])
    yf_t, yb_t = gpu_forward(bank, x, idx, w, c["k"], 0, None)
    monkeypatch.setenv("MOE_GEMV_INBLOCK", "1")
    yf_i, yb_i = gpu_forward(bank, x, idx, w, c["k"], 0, None)
    monkeypatch.delenv("MOE_GEMV_INBLOCK")
    assert np.array_equal(yf_t.view(np.uint32), yf_i.view(np.uint32))
    assert np.array_equal(yb_t, yb_i)
    say(f"routed GEMV T={T}: in-block routing matches the sort tables bit for bit")


def prefill_sample_tokens(idx, E, k, n=512, seed=3):
    """Tokens whose pairs sit at the grouped GEMM's tile edges, then seeded
    random tokens up to n. Slots are the stable sort of the pairs by expert;
    an expert's slots form tiles of 128 rows, and a tile holds 1 to 4 blocks
    of 32 rows. For every block count, among full and partial (last) tiles,
    the tokens of a tile's first and last rows and of the rows on each side of
    a 32-row boundary are taken."""
    P = idx.size
    offs, srt = oracle.sort_pairs(idx.ravel(), E)
    picks, by_class = [], {}
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        for r0 in range(lo, hi, 128):
            rows = min(128, hi - r0)
            key = ((rows + 31) // 32, rows == 128)
            by_class.setdefault(key, []).append((r0, rows))
    for key in sorted(by_class):
        tiles = by_class[key]
        for r0, rows in tiles[:: max(1, len(tiles) // 3)][:3]:
            for r in sorted(set([0, rows - 1] + [b for b in (31, 32, 63, 64, 95, 96) if b < rows])):
                picks.append(int(srt[r0 + r]) // k)
    picks = list(dict.fromkeys(picks))
    rng = np.random.default_rng(seed)
    rest = [t for t in rng.permutation(P // k).tolist() if t not in set(picks)]
    return np.array(sorted(picks + rest[: max(0, n - len(picks))])), sorted(by_class)


def test_forward_prefill_full_shape(big_bank):
    # The prefill workload (8192 tokens, 65,536 pairs on the grouped GEMM):
    # 512 tokens against the oracle, chosen to cover tile edges of every
    # 32-row-block count plus seeded random tokens; then all 8192 tokens
    # against the routed GEMV on the same inputs (that path is itself held to
    # the oracle), which covers every tile row and k step at full shape.
    bank, _ = big_bank
    c = W.CONFIGS["prefill"]
    x, _, logits = W.inputs("prefill")
    idx, w = oracle.route_topk(logits, c["k"])
    say("prefill forward on the GPU (grouped GEMM)")
    yf, yb = gpu_forward(bank, x, idx, w, c["k"])
    assert np.isfinite(yf).all()
    sample, classes = prefill_sample_tokens(idx, c["E"], c["k"])
    say(f"prefill oracle sample: {len(sample)} tokens, tile classes (32-row blocks, full) {classes}")
    recs = host_records(c["bank_seed"], np.unique(idx[sample]), c["H"], c["I"])
    ref_f, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x[sample], idx[sample], w[sample])
    check_f32(yf[sample], ref_f, f"prefill {len(sample)} tokens vs oracle")
    check_bf16_of(yb, yf, "prefill bf16, all tokens")
    say("prefill forward on the GPU (routed GEMV, forced)")
    gf, _ = gpu_forward(bank, x, idx, w, c["k"], wq.MOE_FORCE_DECODE)
    # Two f32 paths round some bf16 mids differently (their gate/up sums
    # differ in the last bits), and a mid that rounds the other way moves a
    # whole output row by one bf16 ulp of that mid times the down weights: the
    # paths agree to the layer tolerance in L2, element by element within twice
    # the per-element bound, and the tokens where they differ most are held to
    # the oracle on both paths.
    rms = np.sqrt(np.mean(gf.astype(np.float64) ** 2))
    diff = np.abs(yf.astype(np.float64) - gf)
    rel = np.linalg.norm(diff) / np.linalg.norm(gf.astype(np.float64))
    worst = np.argsort(diff.max(axis=1))[-16:]
    say(f"grouped GEMM vs routed GEMV, all tokens: rel L2 {rel:.3e}, max |diff|/rms {diff.max() / rms:.3e}, "
        f"worst tokens {sorted(worst.tolist())}")
    assert rel <= 5e-3 and diff.max() <= 2e-2 * rms
    recs = host_records(c["bank_seed"], np.unique(idx[worst]), c["H"], c["I"])
    ref_w, _ = oracle.moe_forward(recs, c["E"], c["H"], c["I"], x[worst], idx[worst], w[worst])
    check_f32(yf[worst], ref_w, "grouped GEMM, 16 most-disagreeing tokens vs oracle")
    check_f32(gf[worst], ref_w, "routed GEMV, 16 most-disagreeing tokens vs oracle")


def test_status_flags_expert_outside_range(tiny_bank):
    # The runtime rule for idx: an expert outside [0, E) is a caller error;
    # the pair contributes nothing and the kernels set MOE_STATUS_BAD_IDX in
    # the workspace's status word, on each path (one-item-per-wave kernels,
    # routed GEMV, grouped GEMM). Valid calls leave the word at 0.
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    recs = host_records(c["bank_seed"], range(E), H, I)
    for T, flags in [(3, 0), (20, 2), (40, 4)]:
        x = synth.activations(500 + T, T, H)
        lg = np.random.default_rng(T).normal(size=(T, E)).astype(np.float32)
        idx, w = oracle.route_topk(lg, k)
        ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, k, H, I, E))
        xd = bf16_tensor(x)
        yf = torch.empty((T, H), dtype=torch.float32, device=DEV)
        wd = torch.from_numpy(w).to(DEV)
        wq.moe_nvfp4_forward(bank, xd, T, torch.from_numpy(idx).to(DEV), wd, k, None, yf, flags | wq.MOE_F32_OUT, ws)
        assert wq.moe_status_read(ws) == 0, (T, flags)
        bad = idx.copy()
        bad[0, 1], bad[T - 1, 0] = E, -7  # one past the end, and negative
        wq.moe_nvfp4_forward(bank, xd, T, torch.from_numpy(bad).to(DEV), wd, k, None, yf, flags | wq.MOE_F32_OUT, ws)
        st = wq.moe_status_read(ws)
        assert st == wq.MOE_STATUS_BAD_IDX, (T, flags, st)
        # the oracle without those pairs: same experts, routing weight 0
        w0 = w.copy()
        w0[0, 1] = w0[T - 1, 0] = 0.0
        ref_f, _ = oracle.moe_forward(recs, E, H, I, x, idx, w0)
        check_f32(yf.cpu().numpy(), ref_f, f"bad idx T={T} flags={flags}")
        wq.moe_status_clear(ws)
        assert wq.moe_status_read(ws) == 0


def test_layer_route_giveup_contract(tiny_bank, monkeypatch):
    # The one-token layer's bounded wait, forced to give up from the host
    # (MOE_DEBUG_ROUTE_GIVEUP: the router workgroups withhold their logits and
    # the waits stop after a few polls; every kernel ends normally): the
    # status word has MOE_STATUS_ROUTE_TIMEOUT, idx is -1, w is 0 and y is the
    # residual. The same workspace then serves a normal call.
    bank, _ = tiny_bank
    c = W.CONFIGS["tiny"]
    H, E = c["H"], c["E"]
    x, Wr, _ = W.inputs("tiny")
    x1 = x[:1]
    res = synth.activations(606, 1, H)
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(1, 2, bank.H, bank.I, bank.E))
    xd, rd = bf16_tensor(x1), bf16_tensor(res)
    wrd = torch.from_numpy(np.ascontiguousarray(Wr)).to(DEV)
    lg = torch.empty((1, E), dtype=torch.float32, device=DEV)
    idx = torch.zeros((1, 2), dtype=torch.int32, device=DEV)
    w = torch.ones((1, 2), dtype=torch.float32, device=DEV)
    yf = torch.empty((1, H), dtype=torch.float32, device=DEV)
    yb = torch.empty((1, H), dtype=torch.int16, device=DEV)
    monkeypatch.setenv("MOE_DEBUG_ROUTE_GIVEUP", "1")
    wq.moe_nvfp4_layer(bank, xd, wrd, 1, 2, rd, lg, idx, w, yf, wq.MOE_F32_OUT, ws)
    wq.moe_nvfp4_layer(bank, xd, wrd, 1, 2, rd, lg, idx, w, yb, 0, ws)
    st = wq.moe_status_read(ws)
    monkeypatch.delenv("MOE_DEBUG_ROUTE_GIVEUP")
    assert st == wq.MOE_STATUS_ROUTE_TIMEOUT, st
    assert idx.cpu().numpy().tolist() == [[-1, -1]]
    assert w.cpu().numpy().tolist() == [[0.0, 0.0]]
    rv = oracle.bf16_to_f32(res).astype(np.float32)
    assert np.array_equal(yf.cpu().numpy(), rv)
    assert np.array_equal(oracle.bf16_to_f32(to_np_bits(yb)), rv)
    say("layer give-up: status, idx, w and y as documented")
    wq.moe_status_clear(ws)
    check_layer_call(bank, "tiny after a give-up", x1, Wr, 2, residual=res, ws=ws)


def test_layer_call_token_counts():
    # the one-call layer for 2..16 tokens (few-token kernels up to 9, the
    # routed GEMV above; 16 keys per lane in the top-k at E = 600), one
    # workspace over calls of several T, each call against route + forward
    H, I = 128, 64
    for E, k, Ts in ((256, 8, (2, 5, 9, 16)), (600, 4, (3, 16))):
        say(f"layer call: E={E}, T in {Ts}")
        bank, _ = W.build_bank(7, H, I, E)
        Wr = synth.router_weights(8, H, E)
        ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(16, k, H, I, E))
        for T in Ts:
            x = synth.activations(90 + T, T, H)
            res = synth.activations(190 + T, T, H) if T % 2 else None
            check_layer_call(bank, f"layer call E={E} T={T}", x, Wr, k, residual=res, ws=ws)


def test_forward_deterministic(big_bank):
    bank, _ = big_bank
    c = W.CONFIGS["batched"]
    x, _, logits = W.inputs("batched", 1)
    idx, w = oracle.route_topk(logits, c["k"])
    a, _ = gpu_forward(bank, x, idx, w, c["k"], 2)
    b, _ = gpu_forward(bank, x, idx, w, c["k"], 2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    p, _ = gpu_forward(bank, x, idx, w, c["k"], 4)
    q, _ = gpu_forward(bank, x, idx, w, c["k"], 4)
    assert np.array_equal(p.view(np.uint32), q.view(np.uint32))


# ---- S8 / S9 -------------------------------------------------------------------------------
def test_affine8_and_rmsnorm():
    # (8, 128, 4100): 17-row workgroups on a 256-CU device, the last with 3 rows
    for T, K, N in [(8, 5120, 5120), (3, 256, 192), (1, 64, 64), (13, 512, 100), (8, 128, 4100)]:
        v = synth.resident_weights(11, N, K)
        codes, scales, biases = oracle.q8_quantize(v)
        x = synth.activations(12, T, K)
        ref_f, ref_b = oracle.affine8_linear(x, codes, scales, biases)
        y = torch.empty((T, N), dtype=torch.int16, device=DEV)
        wq.affine8_g64_linear(bf16_tensor(x), torch.from_numpy(codes.view(np.int32)).to(DEV),
                              bf16_tensor(scales), bf16_tensor(biases), T, K, N, y)
        torch.cuda.synchronize()
        check_bf16(to_np_bits(y), ref_f, f"affine8 {T}x{K}x{N}")
    x = synth.activations(13, 8, 5120)
    y = torch.empty((8, 5120), dtype=torch.int16, device=DEV)
    wq.moe_rmsnorm(bf16_tensor(x), 8, 5120, 1e-6, y)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x, 1e-6)
    check_bf16(to_np_bits(y), oracle.bf16_to_f32(ref), "rmsnorm")


@pytest.mark.parametrize("T,K,N", [(8, 5120, 5120), (1, 1024, 100), (5, 2048, 4100), (2, 3072, 33),
                                   (7, 4096, 5120), (8, 6144, 300), (3, 5120, 17)])
def test_affine8_stream_shapes(T, K, N):
    # up to 8 tokens and K a multiple of 1,024 (at most 6,144): the streaming
    # form, activations and scale and bias rows staged in LDS; 4100 rows give
    # 17-row workgroups (the last with 3 rows), 33 and 17 rows a second row
    # block with 1 row or none. Against the oracle, and against the general
    # kernel on the same data (x copied to an offset of 4 bytes, off the
    # streaming form's conditions): at K = 5120 both give wave w the groups
    # 5 w .. 5 w + 4 and add the same terms in the same order, so bit for bit
    v = synth.resident_weights(31, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(32, T, K)
    ref_f, _ = oracle.affine8_linear(x, codes, scales, biases)
    cd, sd, bd = torch.from_numpy(codes.view(np.int32)).to(DEV), bf16_tensor(scales), bf16_tensor(biases)
    y = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(bf16_tensor(x), cd, sd, bd, T, K, N, y)
    flat = torch.zeros(T * K + 8, dtype=torch.int16, device=DEV)
    flat[2:2 + T * K] = bf16_tensor(x).reshape(-1)
    y2 = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(flat[2:2 + T * K].view(T, K), cd, sd, bd, T, K, N, y2)
    torch.cuda.synchronize()
    check_bf16(to_np_bits(y), ref_f, f"affine8 stream {T}x{K}x{N}")
    check_bf16(to_np_bits(y2), ref_f, f"affine8 general {T}x{K}x{N}")
    if K == 5120:
        assert np.array_equal(to_np_bits(y), to_np_bits(y2)), "streaming and general kernels differ"


def test_affine8_and_rmsnorm_unaligned_rows():
    # activations 4-byte but not 16-byte aligned: the linear stages them with
    # single-word loads, the norm takes its strided loop (also for H not a
    # multiple of 8); 20 tokens take three passes of 8
    T, K, N = 20, 640, 72
    v = synth.resident_weights(21, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(22, T, K)
    ref_f, _ = oracle.affine8_linear(x, codes, scales, biases)
    flat = torch.zeros(T * K + 8, dtype=torch.int16, device=DEV)
    flat[2:2 + T * K] = bf16_tensor(x).reshape(-1)
    xv = flat[2:2 + T * K].view(T, K)
    assert xv.data_ptr() % 16 == 4
    y = torch.empty((T, N), dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(xv, torch.from_numpy(codes.view(np.int32)).to(DEV), bf16_tensor(scales),
                          bf16_tensor(biases), T, K, N, y)
    torch.cuda.synchronize()
    check_bf16(to_np_bits(y), ref_f, f"affine8 unaligned {T}x{K}x{N}")
    for H in (640, 300):
        xr = synth.activations(23, 5, H)
        flat = torch.zeros(5 * H + 8, dtype=torch.int16, device=DEV)
        flat[2:2 + 5 * H] = bf16_tensor(xr).reshape(-1)
        yr = torch.empty((5, H), dtype=torch.int16, device=DEV)
        wq.moe_rmsnorm(flat[2:2 + 5 * H].view(5, H), 5, H, 1e-6, yr)
        torch.cuda.synchronize()
        check_bf16(to_np_bits(yr), oracle.bf16_to_f32(oracle.rmsnorm(xr, 1e-6)), f"rmsnorm unaligned H={H}")


@pytest.mark.parametrize("T,K,N", [(300, 256, 200), (64, 128, 64), (129, 512, 130), (96, 1088, 200),
                                   (40, 5120, 256)])
def test_affine8_gemm_ragged(T, K, N):
    # from 33 tokens the linear runs as the MFMA GEMM: ragged token and row
    # tiles, K of 2 to 8 groups; 96 x 1088 x 200 (two tiles, 17 groups) splits
    # K into three ranges of whole 8-group blocks, the last holding one group;
    # 40 tokens (one tile of 128 rows, 40 real) over 80 groups in ten ranges
    v = synth.resident_weights(14, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(15, T, K)
    ref_f, _ = oracle.affine8_linear(x, codes, scales, biases)
    y = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(bf16_tensor(x), torch.from_numpy(codes.view(np.int32)).to(DEV),
                          bf16_tensor(scales), bf16_tensor(biases), T, K, N, y)
    torch.cuda.synchronize()
    check_bf16(to_np_bits(y), ref_f, f"affine8 gemm {T}x{K}x{N}")


@pytest.mark.parametrize("T,K,N", [(300, 1024, 200), (129, 512, 130), (64, 5120, 384)])
def test_affine8_gemm_dma_form_matches_register_form(T, K, N):
    # K a multiple of 512 with 16-byte aligned scale and bias rows takes the
    # HBM -> LDS form; the same scales and biases copied to an offset of 2
    # bytes take the register form. Both run the same operations in the same
    # order: bit for bit, and within the oracle's bound
    v = synth.resident_weights(24, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(25, T, K)
    ref_f, _ = oracle.affine8_linear(x, codes, scales, biases)
    cd, xd = torch.from_numpy(codes.view(np.int32)).to(DEV), bf16_tensor(x)
    sd, bd = bf16_tensor(scales), bf16_tensor(biases)
    G = K // 64
    sflat = torch.zeros(N * G + 8, dtype=torch.int16, device=DEV)
    bflat = torch.zeros(N * G + 8, dtype=torch.int16, device=DEV)
    sflat[1:1 + N * G] = sd.reshape(-1)
    bflat[1:1 + N * G] = bd.reshape(-1)
    s2, b2 = sflat[1:1 + N * G].view(N, G), bflat[1:1 + N * G].view(N, G)
    assert s2.data_ptr() % 16 == 2 and sd.data_ptr() % 16 == 0
    y = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    y2 = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(xd, cd, sd, bd, T, K, N, y)
    wq.affine8_g64_linear(xd, cd, s2, b2, T, K, N, y2)
    torch.cuda.synchronize()
    check_bf16(to_np_bits(y), ref_f, f"affine8 gemm dma form {T}x{K}x{N}")
    assert np.array_equal(to_np_bits(y), to_np_bits(y2)), "HBM -> LDS and register forms differ"


@pytest.mark.parametrize("T", [256, 1024])
def test_affine8_gemm_full_shape_sampled(T):
    # a 5120 x 5120 resident over 1,024 tokens (8 token tiles x 40 row tiles)
    # and over 256 (2 x 40 tiles: K split into five ranges, partial sums added
    # in range order); the oracle on sampled tokens, every output row
    K, N = 5120, 5120
    v = synth.resident_weights(16, N, K)
    codes, scales, biases = oracle.q8_quantize(v)
    x = synth.activations(17, T, K)
    y = torch.empty((T, N), dtype=torch.int16, device=DEV)
    wq.affine8_g64_linear(bf16_tensor(x), torch.from_numpy(codes.view(np.int32)).to(DEV),
                          bf16_tensor(scales), bf16_tensor(biases), T, K, N, y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, T // 2 - 1, T - 1], np.random.default_rng(18).integers(0, T, 18)]))
    ref_f, _ = oracle.affine8_linear(x[rows], codes, scales, biases)
    check_bf16(to_np_bits(y)[rows], ref_f, f"affine8 gemm {T}x5120x5120 sampled")


# ---- the stacked decode workload: 12 chained layers ------------------------------------
def check_state(got_bits, ref_bits, what):
    """A bf16 layer state h_l of the chain. The single-layer bound (relative L2
    5e-3, per element 1e-2 rms) plus, per element, one bf16 ulp of the
    reference: both sides round the state to bf16 once per layer, and an f32
    result within the layer bound can round to the neighbouring bf16 value."""
    got = oracle.bf16_to_f32(got_bits).astype(np.float64)
    ref = oracle.bf16_to_f32(ref_bits).astype(np.float64)
    rms = np.sqrt(np.mean(ref**2))
    a = np.maximum(np.abs(ref), 2.0**-126)
    ulp = 2.0 ** (np.floor(np.log2(a)) - 7)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    bad = err > 1e-2 * rms + ulp
    say(f"{what}: rel L2 {rel:.3e}, max (|err| - ulp)/rms {np.max(err - ulp) / rms:.3e}")
    assert rel <= 5e-3 and not bad.any(), (what, rel, int(bad.sum()))


def test_stacked_layers_full_shape():
    """The stacked decode workload at full shape: 12 layers, each with its own
    bank of 256 records (3,072 records, 68 GB), its own resident affine8_g64
    linear and router, T = 8, residual added per layer. The oracle's run of
    the whole chain is stored by tests/golden/make_stacked.py (oracle and
    seeded generators only).

    Every layer l is checked on the oracle's own state h_l (h_0 is the
    generated input): the device's RMSNorm of h_l and its affine8 linear of the
    oracle's normalized state (check_bf16), its router logits on the oracle's
    a_l (1e-5 rms) and its top-k of those logits (the oracle's set, order
    checked on the oracle's logits), then the layer on the oracle's a_l and
    routing with h_l as the residual, against the oracle's h_l+1
    (check_state), and the last layer's f32 output (check_f32). A run of the
    device chain on its own state is not compared element by element: on this
    synthetic workload the relative difference between two correct chains
    roughly doubles per layer (the SwiGLU product is quadratic in a_l and each
    layer adds more than the residual carries), so no fixed tolerance holds
    after a few layers."""
    import os

    g = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "stacked_chain.npz"))
    c = W.CONFIGS["stacked"]
    H, I, E, k, T, L = c["H"], c["I"], c["E"], c["k"], c["T"], c["layers"]
    say(f"building the stacked banks: {L} x {E} records")
    banks = [W.build_bank(c["bank_seed"], H, I, E, expert0=l * E) for l in range(L)]
    for l in range(L):
        h = synth.activations(c["seed"], T, H) if l == 0 else g["h"][l - 1]
        n_ref = oracle.rmsnorm(h, 1e-6)
        nd = torch.empty((T, H), dtype=torch.int16, device=DEV)
        wq.moe_rmsnorm(bf16_tensor(h), T, H, 1e-6, nd)
        torch.cuda.synchronize()
        check_bf16(to_np_bits(nd), oracle.bf16_to_f32(n_ref), f"stacked layer {l} rmsnorm")
        codes, scales, biases = oracle.q8_quantize(synth.resident_weights(c["seed"], H, H, layer=l))
        af_ref, a_ref = oracle.affine8_linear(n_ref, codes, scales, biases)
        ad = torch.empty((T, H), dtype=torch.int16, device=DEV)
        wq.affine8_g64_linear(bf16_tensor(n_ref), torch.from_numpy(codes.view(np.int32)).to(DEV),
                              bf16_tensor(scales), bf16_tensor(biases), T, H, H, ad)
        torch.cuda.synchronize()
        check_bf16(to_np_bits(ad), af_ref, f"stacked layer {l} affine8")
        ref_lg = g["logits"][l]
        lg, idx, _ = gpu_route(a_ref, synth.router_weights(c["seed"], H, E, layer=l), None, E, k)
        rms = np.sqrt(np.mean(ref_lg.astype(np.float64) ** 2))
        assert np.max(np.abs(lg.astype(np.float64) - ref_lg)) <= 1e-5 * rms, (l, "router logits")
        # the smallest top-k gap of this workload (4.8e-4) is far above the 2e-5 logit bound
        assert np.all(g["gap"][l] > 2e-5 * rms), l
        assert all(set(idx[t]) == set(g["idx"][l][t]) for t in range(T)), (l, "top-k set")
        _, idx2, w2 = gpu_route(a_ref, None, ref_lg, E, k)
        assert np.array_equal(idx2, g["idx"][l]), (l, "top-k")
        check_weights(w2, g["w"][l], np.take_along_axis(ref_lg, g["idx"][l], axis=1))
        yf, yb = gpu_forward(banks[l][0], a_ref, g["idx"][l], g["w"][l], k, residual=h)
        check_state(yb, g["h"][l], f"stacked layer {l}")
        check_bf16_of(yb, yf, f"stacked layer {l} bf16")
    check_f32(yf, g["y_last_f32"], "stacked last layer f32")
    del banks
    torch.cuda.empty_cache()
