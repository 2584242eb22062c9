"""Pins for the oracle's per-layer functions (CPU only): RMSNorm, RoPE, attention, SwiGLU."""
import math

import numpy as np
import pytest

import oracle
import synth


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_form_and_invariants():
    d = 48
    g = 1.0 + synth.normal(3, (d,))
    c = 0.37
    y = oracle.rmsnorm(np.full((1, d), c), g, 1e-6)
    assert np.allclose(y[0], c / math.sqrt(c * c + 1e-6) * g.astype(np.float64), rtol=1e-14)
    x = synth.normal(4, (5, d), scale=1.0).astype(np.float64)
    y1 = oracle.rmsnorm(x, np.ones(d), 0.0)
    assert np.allclose(np.sqrt(np.mean(y1 ** 2, axis=1)), 1.0, rtol=1e-13)
    assert np.allclose(oracle.rmsnorm(7.5 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-13)
    # scalar re-derivation of one row with epsilon inside the root
    row = x[2]
    ms = sum(v * v for v in row) / d
    ref = [v / math.sqrt(ms + 1e-6) * float(gg) for v, gg in zip(row, g)]
    assert np.allclose(oracle.rmsnorm(x[2:3], g, 1e-6)[0], ref, rtol=1e-13)


# ----------------------------------------------------------------------------- RoPE

def test_rope_hand_example_rotate_half_pairing():
    # hd = 4, theta = 10000: pairs (0, 2) at omega 1 and (1, 3) at omega 0.01
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]], np.float32)
    c, s = oracle.rope_table(2, 4, 10000.0)
    out = oracle.rope_apply_f32(x, c[1:2], s[1:2])[0, 0]
    a, b = 1.0, 0.01
    ref = [1 * math.cos(a) - 3 * math.sin(a), 2 * math.cos(b) - 4 * math.sin(b),
           3 * math.cos(a) + 1 * math.sin(a), 4 * math.cos(b) + 2 * math.sin(b)]
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_rope_position_zero_is_identity_and_table_matches_numpy():
    c, s = oracle.rope_table(300, 64, 1e6)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    x = synth.normal(5, (1, 3, 64), scale=1.0)
    assert np.array_equal(oracle.rope_apply_f32(x, c[:1], s[:1]), x)
    i = np.arange(32, dtype=np.float64)
    ang = np.arange(300, dtype=np.float64)[:, None] * np.power(1e6, -2.0 * i / 64)[None, :]
    for ref, tab in ((np.cos(ang), c), (np.sin(ang), s)):
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(tab.astype(np.float64) - ref) <= ulp)


def test_rope_f32_matches_f64_rotation_and_preserves_pair_norms():
    hd, n = 128, 40
    pos = np.arange(1000, 1000 + n)
    c, s = oracle.rope_table(1100, hd, 1e6)
    x = synth.normal(6, (n, 5, hd), scale=1.0)
    y32 = oracle.rope_apply_f32(x, c[pos], s[pos]).astype(np.float64)
    y64 = oracle.rope_apply(x, pos, hd, 1e6)
    assert np.max(np.abs(y32 - y64)) < 2e-6 * np.max(np.abs(x))
    h = hd // 2
    n_in = x[..., :h].astype(np.float64) ** 2 + x[..., h:].astype(np.float64) ** 2
    n_out = y64[..., :h] ** 2 + y64[..., h:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)


def test_rope_relative_position_identity():
    hd = 64
    q = synth.normal(8, (1, 1, hd), scale=1.0).astype(np.float64)
    k = synth.normal(9, (1, 1, hd), scale=1.0).astype(np.float64)
    for m, n in [(5, 2), (1000, 37), (58000, 57999)]:
        lhs = np.sum(oracle.rope_apply(q, [m], hd, 1e6) * oracle.rope_apply(k, [n], hd, 1e6))
        rhs = np.sum(oracle.rope_apply(q, [m - n], hd, 1e6) * k)
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


# ----------------------------------------------------------------------------- attention

def brute_attention(q, K, V, positions):
    n, Hq, hd = q.shape
    G = Hq // K.shape[1]
    out = np.zeros((n, Hq, hd))
    for i in range(n):
        for h in range(Hq):
            g = h // G
            sc = [sum(float(q[i, h, e]) * float(K[j, g, e]) for e in range(hd)) / math.sqrt(hd)
                  for j in range(positions[i] + 1)]
            m = max(sc)
            w = [math.exp(v - m) for v in sc]
            z = sum(w)
            for e in range(hd):
                out[i, h, e] = sum(w[j] * float(V[j, g, e]) for j in range(len(w))) / z
    return out


@pytest.mark.parametrize("Hq,Hkv,hd,D,n", [(4, 2, 8, 3, 5), (6, 2, 8, 0, 4), (2, 2, 16, 9, 3)])
def test_attention_matches_brute_force(Hq, Hkv, hd, D, n):
    T = D + n
    q = synth.normal(20, (n, Hq, hd), scale=1.0)
    K = synth.normal(21, (T + 4, Hkv, hd), scale=1.0)
    V = synth.normal(22, (T + 4, Hkv, hd), scale=1.0)
    pos = np.arange(D, D + n)
    got = oracle.attention(q, K, V, pos)
    assert np.allclose(got, brute_attention(q, K, V, pos), rtol=1e-12, atol=1e-13)


def test_attention_single_visible_key_and_causality():
    q = synth.normal(30, (6, 4, 16), scale=1.0)
    K = synth.normal(31, (6, 2, 16), scale=1.0)
    V = synth.normal(32, (6, 2, 16), scale=1.0)
    pos = np.arange(6)
    o = oracle.attention(q, K, V, pos)
    assert np.allclose(o[0, 0], V[0, 0]) and np.allclose(o[0, 3], V[0, 1])
    # rows beyond a query's position must not matter
    K2, V2 = K.copy(), V.copy()
    K2[4:] = 123.0
    V2[4:] = -7.0
    o2 = oracle.attention(q[:4], K2, V2, pos[:4])
    assert np.array_equal(o2, o[:4])


def test_gqa_with_duplicated_kv_heads_equals_multi_head():
    Hq, Hkv, hd, n = 6, 2, 8, 7
    G = Hq // Hkv
    q = synth.normal(40, (n, Hq, hd), scale=1.0)
    K = synth.normal(41, (n, Hkv, hd), scale=1.0)
    V = synth.normal(42, (n, Hkv, hd), scale=1.0)
    pos = np.arange(n)
    gqa = oracle.attention(q, K, V, pos)
    mha = oracle.attention(q, np.repeat(K, G, axis=1), np.repeat(V, G, axis=1), pos)
    assert np.allclose(gqa, mha, rtol=1e-14)


# ----------------------------------------------------------------------------- SwiGLU

def test_swiglu_closed_form():
    y = np.array([[0.5, -1.25]])
    Wg = np.array([[1.0, 2.0]])
    Wu = np.array([[-0.5, 0.25]])
    Wd = np.array([[2.0], [-3.0]])
    g = 0.5 * 1.0 + -1.25 * 2.0
    u = 0.5 * -0.5 + -1.25 * 0.25
    h = g / (1.0 + math.exp(-g)) * u
    assert np.allclose(oracle.swiglu_ffn(y, Wg, Wu, Wd)[0], [2.0 * h, -3.0 * h], rtol=1e-14)
    assert np.all(oracle.swiglu_ffn(np.zeros((2, 2)), Wg, Wu, Wd) == 0.0)


def test_cache_rows_f16_rne_and_q8_0():
    x = np.array([[[1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 6.0e-8, 65504.0]]], np.float32)
    f = oracle.cache_encode_rows(x, "f16")
    assert f.dtype == np.float16
    assert [float(v) for v in f[0, 0]] == [1.0, 1.0 + 2.0 ** -9, 5.960464477539063e-08, 65504.0]
    rows = synth.normal(50, (3, 2, 64), scale=1.0)
    d16, q = oracle.cache_encode_rows(rows, "q8_0")
    assert d16.shape == (3, 2, 2) and q.shape == (3, 2, 2, 32)
    back = oracle.cache_decode_rows((d16, q), "q8_0")
    assert back.shape == rows.shape and np.max(np.abs(back - rows)) < 0.02


# ----------------------------------------------------------------------- fp16 operands

def test_to_f16_round_to_nearest_even_and_saturation():
    """binary16 has 10 fraction bits: the spacing at 1 is 2^-10, the largest finite value
    is 65504, the smallest subnormal 2^-24; halfway cases go to the even neighbour."""
    f = oracle.to_f16
    assert f(1 + 2.0 ** -11) == 1.0                       # tie -> even (1.0)
    assert f(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9         # tie -> even (1 + 2 * 2^-10)
    assert f(1 + 2.0 ** -11 + 2.0 ** -30) == 1 + 2.0 ** -10
    assert f(-(1 + 2.0 ** -11 + 2.0 ** -30)) == -(1 + 2.0 ** -10)
    assert f(65519.0) == 65504.0                          # below the overflow midpoint
    with np.errstate(over="ignore"):
        assert np.isinf(f(65520.0))                       # at it: rounds to infinity
    assert f(1e6, saturate=True) == 65504.0 and f(-1e6, saturate=True) == -65504.0
    assert f(2.0 ** -24) == 2.0 ** -24                    # smallest subnormal
    assert f(2.0 ** -25) == 0.0                           # tie -> even (0)
    assert f(3 * 2.0 ** -25) == 2.0 ** -23                # tie -> even (2 * 2^-24)
    x = synth.normal(50, (4096,), scale=3.0).astype(np.float64)
    r = f(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -11 + 2.0 ** -25)


def test_attention_f16_weights_exact_at_powers_of_two_and_bounded_otherwise():
    """p_f16 rounds exp(s - max) to binary16.  With scores at integer multiples of ln 2
    the weights are powers of two (exact in binary16) and the result is the exact one; with
    random scores it stays within binary16 rounding (2^-11 relative per weight) of it."""
    n, hd = 6, 4
    ks = np.array([0, -1, -3, -2, -5, -4, -7, -6, -1, -2], dtype=np.float64)[:n]
    K = np.zeros((n, 1, hd))
    K[:, 0, 0] = ks * math.log(2.0)
    q = np.zeros((n, 1, hd))
    q[:, 0, 0] = math.sqrt(hd)                            # s_j = q . K_j / sqrt(hd) = k_j ln 2
    V = synth.normal(51, (n, 1, hd), scale=1.0).astype(np.float64)
    pos = np.arange(n)
    a = oracle.attention(q, K, V, pos)
    b = oracle.attention(q, K, V, pos, p_f16=True)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    q = synth.normal(52, (9, 2, 8), scale=2.0).astype(np.float64)
    K = synth.normal(53, (9, 2, 8), scale=2.0).astype(np.float64)
    V = synth.normal(54, (9, 2, 8), scale=1.0).astype(np.float64)
    pos = np.arange(9)
    a = oracle.attention(q, K, V, pos)
    b = oracle.attention(q, K, V, pos, p_f16=True)
    bound = 2 * 2.0 ** -11 * np.max(np.abs(V))
    assert 0 < np.max(np.abs(a - b)) <= bound


def test_swiglu_f16_intermediate_saturates_and_rounds():
    y = np.array([[1.0, 2.0]])
    Wg = np.array([[100.0, 0.0], [1.0, 0.0]])             # gate: 100, 1
    Wu = np.array([[0.0, 400.0], [0.0, 1.0 / 3.0]])       # up: 800, 2/3
    Wd = np.eye(2)
    h = oracle.swiglu_ffn(y, Wg, Wu, Wd, h_f16=True)
    # silu(100) * 800 = 80000 (saturated to 65504); silu(1) * 2/3 rounded to binary16
    s1 = 1.0 / (1.0 + math.exp(-1.0)) * (2.0 / 3.0)
    assert h[0, 0] == 65504.0
    assert h[0, 1] == float(np.float16(s1)) and h[0, 1] != s1
