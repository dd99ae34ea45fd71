"""Pins of the pack-side oracle: the global g recovered from weight_scale_2
("Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit residents",
"What this pack holds", global-scales bullet), and the library's host
implementation against it (no GPU needed: the library's function runs on the
host). The record digests are checked on the GPU in test_gpu_parity.py. Also
the expert cache's placement rule (oracle.lru_slots), pinned by a hand-worked
example and invariants."""
import ctypes as C

import numpy as np
import pytest

import oracle
import weight_quantized_moe_amd as wq

DIV = np.float32(2688.0)


def image(g):
    return (np.asarray(g, dtype=np.float32) / DIV).astype(np.float32)


def log_uniform(rng, n, lo=1e-7, hi=1e4):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.float32)


def test_representable_scales_are_exact():
    # every f32(g / 2688) has a g: the oracle must find one (flag 0) whose image
    # is that value
    rng = np.random.default_rng(1)
    g_src = log_uniform(rng, 20000, 1e-3, 1e7)
    ws2 = image(g_src)
    g, inexact = oracle.global_from_ws2(ws2)
    assert not inexact.any()
    assert np.array_equal(image(g), ws2)


def test_brute_force_neighbourhood():
    # the rule by exhaustive search over 601 neighbours of the rounded product
    # (a different method from the oracle's bisection)
    rng = np.random.default_rng(2)
    ws2 = log_uniform(rng, 3000)
    target = ws2.astype(np.float64) * 2688.0
    centre = target.astype(np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-300, 301, dtype=np.int64)
    cand_bits = centre[:, None] + offs[None, :]
    cand = cand_bits.astype(np.uint32).view(np.float32)
    err = np.abs(image(cand).astype(np.float64) - ws2.astype(np.float64)[:, None])
    dist = np.abs(cand.astype(np.float64) - target[:, None])
    order = np.lexsort((cand_bits & 1, dist, err), axis=1)  # err first, then dist, then even
    pick = cand[np.arange(len(ws2)), order[:, 0]]
    exact = err.min(axis=1) == 0
    g, inexact = oracle.global_from_ws2(ws2)
    assert np.array_equal(g.view(np.uint32), pick.view(np.uint32))
    assert np.array_equal(inexact == 0, exact)


def test_inexact_rate_closed_form():
    # For g = ws2 * 2688, ulp(g) is 2^12 ulp(ws2) when ws2's significand is at
    # least 4096/2688 = 1.5238 and 2^11 ulp(ws2) below it. Consecutive g then
    # step 4096/2688 ulps of ws2 in the upper part (a fraction 1 - 2688/4096 =
    # 11/32 of those ws2 have no g) and 2048/2688 < 1 ulp in the lower part
    # (every ws2 has one). For log-uniform ws2 the upper part is
    # log2(2688/2048) of each binade, so the rate is log2(1.3125) * 11/32 =
    # 0.13486. (The pages report 4,878 of 37,632 projections, 12.96 %, for the
    # release's own scales.)
    rng = np.random.default_rng(3)
    ws2 = log_uniform(rng, 400000)
    _, inexact = oracle.global_from_ws2(ws2)
    expect = np.log2(2688.0 / 2048.0) * 11.0 / 32.0
    assert abs(inexact.mean() - expect) < 0.003, (inexact.mean(), expect)
    # and no inexact value in the lower part of a binade
    sig = np.frexp(ws2.astype(np.float64))[0] * 2.0  # significand in [1, 2)
    assert not inexact[sig < 4096.0 / 2688.0 - 1e-6].any()


def test_stored_g_within_one_ulp():
    # the pages: the stored g is about one f32 ulp (7e-8 relative) from the
    # exact value at worst
    rng = np.random.default_rng(4)
    ws2 = log_uniform(rng, 50000)
    g, inexact = oracle.global_from_ws2(ws2)
    target = ws2.astype(np.float64) * 2688.0
    ulp = np.spacing(g).astype(np.float64)
    assert np.all(np.abs(g.astype(np.float64) - target) <= ulp)
    # inexact ones: the image is one ulp of ws2 away, on one side or the other
    img = image(g)
    off = np.abs(img.view(np.int32).astype(np.int64) - ws2.view(np.int32).astype(np.int64))
    assert np.all(off[inexact == 1] == 1) and np.all(off[inexact == 0] == 0)


def test_library_matches_oracle():
    rng = np.random.default_rng(5)
    edge = np.array([np.finfo(np.float32).tiny, np.float32(1e-40), np.float32(1.4e-45), 1.0, 2.0, 0.5,
                     np.float32(3.4028234e38 / 2688.0), np.float32(1.5238095), np.float32(1.5238096),
                     np.float32(1.0 / 2688.0)], dtype=np.float32)
    ws2 = np.concatenate([edge, log_uniform(rng, 200000, 1e-30, 1e30)])
    g_ref, f_ref = oracle.global_from_ws2(ws2)
    g, f = wq.moe_nvfp4_global_from_ws2(ws2)
    assert np.array_equal(g.view(np.uint32), g_ref.view(np.uint32))
    assert np.array_equal(f, f_ref)


@pytest.mark.parametrize("bad", [0.0, -1.0, np.inf, np.nan, np.float32(3.4e38)])
def test_library_rejects_bad_scales(bad):
    ws2 = np.array([1.0, bad], dtype=np.float32)
    g = np.full(2, 7.0, dtype=np.float32)
    L = wq.lib()
    rc = L.moe_nvfp4_global_from_ws2(ws2.ctypes.data_as(C.c_void_p), 2, g.ctypes.data_as(C.c_void_p), None)
    assert rc == wq.MOE_EINVAL
    assert np.all(g == 7.0)  # nothing written
    assert L.moe_nvfp4_global_from_ws2(None, -1, None, None) == wq.MOE_EINVAL
    assert L.moe_nvfp4_global_from_ws2(None, 0, None, None) == wq.MOE_OK


# ---- the expert cache's placement rule (oracle.lru_slots) ------------------------------
def test_lru_slots_hand_worked():
    # 3 slots. call 1 fills 0, 1 with experts 7, 8; call 2: 8 hits, 9 takes the
    # empty slot 2; call 3: 7 hits (slot 0), 10 evicts the slot used longest ago
    # among those not named: slot 1 (8, last used in call 2) and slot 2 (9,
    # call 2) tie, the lower slot wins -> slot 1; call 4: 8 misses and takes
    # slot 2 (9, call 2: older than slots 0 and 1, used in call 3)
    got = oracle.lru_slots(3, [[7, 8], [8, 9], [7, 10], [8]])
    assert got == [([0, 1], 0, 2), ([1, 2], 1, 1), ([0, 1], 1, 1), ([2], 0, 1)]


def test_lru_slots_invariants():
    rng = np.random.default_rng(8)
    calls = [list(rng.choice(40, size=rng.integers(1, 6), replace=False)) for _ in range(300)]
    # enough slots for everything: each expert misses exactly once
    out = oracle.lru_slots(40, calls)
    assert sum(m for _, _, m in out) == len({e for c in calls for e in c})
    # a call's experts sit in distinct slots, and a hit keeps its slot
    out = oracle.lru_slots(6, calls)
    where = {}
    for c, (slots, hits, misses) in zip(calls, out):
        assert len(set(slots)) == len(c) and hits + misses == len(c)
        assert hits == sum(1 for e in c if e in where)
        for e, s in zip(c, slots):
            if e in where:
                assert where[e] == s
        for e in list(where):
            if where[e] in slots and e not in c:
                del where[e]
        for e, s in zip(c, slots):
            where[e] = s
    # duplicates inside a call count as hits after the first
    assert oracle.lru_slots(2, [[3, 3, 4]]) == [([0, 0, 1], 1, 2)]
