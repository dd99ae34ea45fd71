"""Pins of the oracle's router, top-k, softmax and pair sort: brute force with
Python's sorted(), a library softmax, and a float64 numpy matmul."""
import numpy as np
import pytest
import scipy.special

import oracle
import synth


def test_router_logits_match_numpy_matmul():
    x = synth.activations(1, 5, 256)
    Wr = synth.router_weights(1, 256, 16)
    got = oracle.router_logits(x, Wr)
    ref = (oracle.bf16_to_f32(x).astype(np.float64) @ Wr.astype(np.float64).T).astype(np.float32)
    # both are f64 sums rounded once to f32; the summation orders differ, so
    # allow one f32 ulp
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got - ref) <= ulp)


def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(16, 2), (256, 8), (8, 8), (5, 1)])
def test_topk_matches_full_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.normal(size=(40, E)).astype(np.float32)
    # ties, and -0 against +0
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0
    lg[2, :] = np.round(lg[2, :])
    lg[3, 1] = lg[3, 2] = lg[3].max()
    idx, w = oracle.route_topk(lg, k)
    for t in range(lg.shape[0]):
        assert idx[t].tolist() == _brute_topk(lg[t], k)
        sel = lg[t, idx[t]].astype(np.float64)
        ref = scipy.special.softmax(sel)
        assert np.all(np.abs(w[t].astype(np.float64) - ref) <= np.spacing(np.float32(ref)))


def test_topk_k1_weight_is_one_and_nan_rejected():
    lg = np.random.default_rng(0).normal(size=(7, 16)).astype(np.float32)
    idx, w = oracle.route_topk(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    lg[3, 4] = np.nan
    with pytest.raises(ValueError):
        oracle.route_topk(lg, 2)
    with pytest.raises(ValueError):
        oracle.route_topk(lg[:, :4], 5)


def test_sort_pairs_matches_stable_sort():
    rng = np.random.default_rng(9)
    for P, E in [(8, 16), (256, 256), (65536, 256), (1, 1), (0, 4)]:
        idx = rng.integers(0, E, P).astype(np.int32)
        off, srt = oracle.sort_pairs(idx, E)
        assert srt.tolist() == sorted(range(P), key=lambda p: int(idx[p]))
        assert off.tolist() == [0] + np.cumsum(np.bincount(idx, minlength=E)).tolist()
    with pytest.raises(ValueError):
        oracle.sort_pairs(np.array([0, 4], np.int32), 4)
