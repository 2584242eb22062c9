"""Pins for the oracle's routed-expert functions (CPU only)."""
import struct

import numpy as np

import oracle
import synth


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def test_router_ordered_matches_scalar_float32_evaluation():
    T, E, d = 3, 5, 64
    y = synth.normal(1, (T, d), scale=1.0)
    w = synth.normal(2, (E, d))
    d16, q = oracle.q8_0_encode(w)
    r = oracle.router_logits_ordered(y, d16, q)
    for t in range(T):
        for e in range(E):
            acc = None
            for b in range(d // 32):
                P = None
                for j in range(32):
                    p = f32(float(q[e, b, j]) * float(y[t, 32 * b + j]))
                    P = p if P is None else f32(P + p)
                term = f32(float(d16[e, b]) * P)
                acc = term if acc is None else f32(acc + term)
            assert r[t, e] == np.float32(acc)
    # close to the plain dot product with the dequantised router
    ref = y.astype(np.float64) @ oracle.q8_0_decode(d16, q).astype(np.float64).T
    assert np.allclose(r, ref, rtol=1e-4, atol=1e-5)


def test_topk_matches_brute_force_sort_with_ties():
    r = synth.uniform(3, (50, 16), -1, 1)
    r[0, :] = 0.25                       # all tied: lowest indices win
    r[1, [3, 7, 9]] = 5.0                # a three-way tie at the top
    idx, w = oracle.moe_route(r, 4)
    for t in range(r.shape[0]):
        ref = sorted(range(16), key=lambda e: (-float(r[t, e]), e))[:4]
        assert list(idx[t]) == ref
    assert list(idx[0]) == [0, 1, 2, 3] and list(idx[1][:3]) == [3, 7, 9]
    assert np.allclose(w.sum(axis=1), 1.0)
    sel = np.take_along_axis(r, idx, 1).astype(np.float64)
    ref_w = np.exp(sel) / np.exp(sel).sum(1, keepdims=True)
    assert np.allclose(w, ref_w, rtol=1e-13)


def test_dominant_logit_and_k1():
    r = np.zeros((2, 8), np.float32)
    r[0, 5] = 80.0
    idx, w = oracle.moe_route(r, 3)
    assert idx[0, 0] == 5 and w[0, 0] >= 1 - 1e-15
    idx1, w1 = oracle.moe_route(synth.uniform(4, (6, 8)), 1)
    assert np.all(w1 == 1.0)


def test_identical_experts_reduce_to_dense_ffn():
    T, d, Fe, E, k = 9, 32, 24, 6, 3
    y = synth.normal(5, (T, d), scale=1.0).astype(np.float64)
    Wg = synth.normal(6, (Fe, d), scale=0.2).astype(np.float64)
    Wu = synth.normal(7, (Fe, d), scale=0.2).astype(np.float64)
    Wd = synth.normal(8, (d, Fe), scale=0.2).astype(np.float64)
    r = synth.uniform(9, (T, E), -2, 2)
    idx, w = oracle.moe_route(r, k)
    moe = oracle.moe_ffn(y, idx, w, np.stack([Wg] * E), np.stack([Wu] * E), np.stack([Wd] * E))
    dense = oracle.swiglu_ffn(y, Wg, Wu, Wd)
    assert np.allclose(moe, dense, rtol=1e-12, atol=1e-14)


def test_moe_sums_in_rank_order_per_token():
    T, d, Fe, E, k = 4, 32, 8, 5, 2
    y = synth.normal(10, (T, d), scale=1.0).astype(np.float64)
    Wg = synth.normal(11, (E, Fe, d), scale=0.3).astype(np.float64)
    Wu = synth.normal(12, (E, Fe, d), scale=0.3).astype(np.float64)
    Wd = synth.normal(13, (E, d, Fe), scale=0.3).astype(np.float64)
    idx, w = oracle.moe_route(synth.uniform(14, (T, E), -1, 1), k)
    got = oracle.moe_ffn(y, idx, w, Wg, Wu, Wd)
    for t in range(T):
        ref = np.zeros(d)
        for rank in range(k):
            e = idx[t, rank]
            ref = ref + w[t, rank] * oracle.swiglu_ffn(y[t:t + 1], Wg[e], Wu[e], Wd[e])[0]
        assert np.allclose(got[t], ref, rtol=1e-13, atol=1e-15)
