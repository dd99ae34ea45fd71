"""The forward that allocates nothing (moe_nvfp4_forward_noalloc), through the
C ABI: on the same inputs it must give exactly what moe_nvfp4_forward gives
with a workspace of its own, on each path (grouped GEMM, routed GEMV,
one-item-per-wave kernels), over successive calls that each leave the shared
scratch behind for the next (the later ones smaller); it reports bad expert
ids in the caller's status word and refuses calls beyond its scratch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W

wq = pytest.importorskip("weight_quantized_moe_amd")
pytestmark = pytest.mark.gpu

DEV = "cuda"
H, I, E, K = 512, 256, 32, 8


@pytest.fixture(scope="module")
def bank():
    return W.build_bank(21, H, I, E)[0]


def _inputs(T, seed):
    x = synth.activations(seed, T, H)
    lg = np.random.default_rng(seed).normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, K)
    return x, idx, w


def _both(bank, x, idx, w, flags, residual=None, status=None):
    T = x.shape[0]
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    idd = torch.from_numpy(idx).to(DEV)
    wd = torch.from_numpy(w).to(DEV)
    rd = None if residual is None else torch.from_numpy(residual.view(np.int16)).to(DEV)
    f32 = flags & wq.MOE_F32_OUT
    ya = torch.empty((T, H), dtype=torch.float32 if f32 else torch.int16, device=DEV)
    yb = torch.empty_like(ya)
    ws = wq.workspace(wq.moe_nvfp4_workspace_bytes(T, K, H, I, E))
    wq.moe_nvfp4_forward(bank, xd, T, idd, wd, K, rd, ya, flags, ws)
    wq.moe_nvfp4_forward_noalloc(bank, xd, T, idd, wd, K, rd, yb, flags, status)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yb.cpu().numpy()


def test_noalloc_matches_forward_on_successive_calls(bank):
    # 200 tokens (1,600 pairs: grouped GEMM), then 20 (routed GEMV), then 3
    # (one-item-per-wave kernels), then 200 again: each call finds the last
    # call's tables and rows in the scratch
    recs = {e: oracle.pack_record(H, I, *W.host_parts(21, e, H, I)) for e in range(E)}
    for n, (T, seed) in enumerate([(200, 1), (20, 2), (3, 3), (200, 4)]):
        x, idx, w = _inputs(T, seed)
        res = synth.activations(seed + 50, T, H) if n % 2 else None
        for flags in (wq.MOE_F32_OUT, 0):
            a, b = _both(bank, x, idx, w, flags, res)
            assert np.array_equal(a.view(np.uint32 if flags else np.uint16), b.view(np.uint32 if flags else np.uint16)), (T, flags)
            if flags:
                ref, _ = oracle.moe_forward(recs, E, H, I, x, idx, w, residual=res)
                rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
                rel = np.linalg.norm(b - ref) / np.linalg.norm(ref)
                assert rel <= 5e-3 and np.max(np.abs(b - ref)) <= 1e-2 * rms, (T, rel)
        print(f"noalloc call {n}: T={T} equal to the workspace forward bit for bit", flush=True)


def test_noalloc_status_and_limit(bank):
    x, idx, w = _inputs(20, 7)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    _both(bank, x, idx, w, wq.MOE_F32_OUT, status=st)
    assert int(st.item()) == 0
    bad = idx.copy()
    bad[3, 2] = E
    _both(bank, x, bad, w, wq.MOE_F32_OUT, status=st)
    assert int(st.item()) == wq.MOE_STATUS_BAD_IDX
    # beyond the scratch: refused before anything is enqueued
    T = 2000
    assert wq.moe_nvfp4_workspace_bytes(T, K, H, I, E) > wq.MOE_NOALLOC_SCRATCH_BYTES
    xd = torch.zeros((T, H), dtype=torch.int16, device=DEV)
    idd = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    wd = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    with pytest.raises(wq.MoeError) as ei:
        wq.moe_nvfp4_forward_noalloc(bank, xd, T, idd, wd, K, None, y, 0)
    assert ei.value.code == wq.MOE_EWORKSPACE
