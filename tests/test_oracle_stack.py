"""Pins for the oracle's layer stack, drivers and serialized state (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.state import HEADER
import synth
from model_inputs import TINY_DENSE, TINY_MOE, q8_layers


def rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("base", [TINY_DENSE, TINY_MOE])
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_chunked_equals_layer_major_and_chunk_sizes_agree(base, kv):
    w = base.with_(kv_type=kv)
    m = oracle.OracleModel(w, q8_layers(w))
    x = synth.prompt_inputs(w)
    ref = m.prefill_layer_major(x)
    for chunk in (1, 3, w.chunk, w.n_prompt):
        got = m.prefill(x, chunk)
        assert rel(got, ref) < 1e-12, chunk
    assert np.all(np.isfinite(ref))


def test_prefix_outputs_do_not_change_when_tokens_are_appended():
    w = TINY_DENSE
    m = oracle.OracleModel(w, q8_layers(w))
    x = synth.prompt_inputs(w)
    full = m.prefill_layer_major(x)
    pre = m.prefill_layer_major(x[:11])
    assert rel(pre, full[:11]) < 1e-12


@pytest.mark.parametrize("base", [TINY_DENSE, TINY_MOE])
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_layer_rows_equals_the_full_layer_at_those_rows(base, kv):
    """The sampled-row evaluation used for long prompts is the full layer restricted to
    the rows, and writes the same cache rows."""
    w = base.with_(kv_type=kv, n_layer=1)
    m = oracle.OracleModel(w, q8_layers(w)[:1])
    x = synth.prompt_inputs(w).astype(np.float64)
    full = m.prefill_layer_major(x)
    rows = [0, 1, 5, w.n_prompt - 2]
    got, cache = m.layer_rows(0, x, rows)
    assert rel(got, full[rows]) < 1e-12
    T = max(rows) + 1
    assert np.array_equal(cache.kval[0][:T], m.last_cache.kval[0][:T])
    assert np.array_equal(cache.vval[0][:T], m.last_cache.vval[0][:T])


def test_layer_by_hand_matches_stack():
    """One layer written out step by step from the dequantised weights."""
    w = TINY_DENSE.with_(n_layer=1)
    layers = q8_layers(w)
    m = oracle.OracleModel(w, layers)
    x = synth.prompt_inputs(w, 9).astype(np.float64)
    out = m.prefill_layer_major(x)
    W = oracle.dequant_layer(layers[0], m.K_of)
    hd, Hq, Hkv = w.head_dim, w.n_head, w.n_kv_head
    y = oracle.rmsnorm(x, W["attn_norm"], w.rms_eps)
    q = (y @ W["wq"].T).reshape(9, Hq, hd)
    k = (y @ W["wk"].T).reshape(9, Hkv, hd)
    v = (y @ W["wv"].T).reshape(9, Hkv, hd)
    pos = np.arange(9)
    q = oracle.rope_apply(q, pos, hd, w.rope_theta)
    k = oracle.rope_apply(k, pos, hd, w.rope_theta)
    k = k.astype(np.float16).astype(np.float64)
    v = v.astype(np.float16).astype(np.float64)
    o = oracle.attention(q, k, v, pos).reshape(9, Hq * hd)
    h = x + o @ W["wo"].T
    y2 = oracle.rmsnorm(h, W["ffn_norm"], w.rms_eps)
    g = y2 @ W["w_gate"].T
    ref = h + ((g / (1 + np.exp(-g))) * (y2 @ W["w_up"].T)) @ W["w_down"].T
    assert rel(out, ref) < 1e-5      # the float32 RoPE / cache rounding is the difference


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_state_round_trip_size_and_continuation(kv):
    w = TINY_DENSE.with_(kv_type=kv)
    m = oracle.OracleModel(w, q8_layers(w))
    x = synth.prompt_inputs(w)
    cache = m.new_cache(40)
    m.prefill(x[:16], 7, cache=cache)
    blob = oracle.state_bytes(cache, w.rope_theta)
    assert len(blob) == oracle.state_size(w.n_layer, w.n_kv_head, w.head_dim, 16, kv)
    assert blob[:4] == b"CPKV"
    c2 = m.new_cache(40)
    oracle.load_state(c2, blob)
    assert oracle.state_bytes(c2, w.rope_theta) == blob
    a = m.prefill(x[16:], 7, cache=cache)
    b = m.prefill(x[16:], 7, cache=c2)
    assert np.array_equal(a, b)


def test_state_header_mutations_rejected():
    w = TINY_DENSE
    m = oracle.OracleModel(w, q8_layers(w))
    cache = m.new_cache(16)
    m.prefill(synth.prompt_inputs(w, 5), 5, cache=cache)
    blob = bytearray(oracle.state_bytes(cache, w.rope_theta))
    for off in (0, 4, 8, 20, 24):
        bad = bytearray(blob)
        bad[off] ^= 0x5A
        with pytest.raises(ValueError):
            oracle.parse_state(bytes(bad))
    with pytest.raises(ValueError):
        oracle.parse_state(bytes(blob[:-1]))
    c3 = oracle.OracleCache(w.n_layer, 16, w.n_kv_head * 2, w.head_dim, "f16")
    with pytest.raises(ValueError):
        oracle.load_state(c3, bytes(blob))


def test_state_sizes_at_workload_geometry():
    # 16 layers x 8 kv heads x 128 dims, K and V
    assert oracle.state_size(16, 8, 128, 17055, "f16") == 1_117_716_512
    assert oracle.state_size(16, 8, 128, 58300, "q8_0") == 2_029_772_832
    assert HEADER.size == 32


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_state_byte_order_at_explicit_offsets(kv):
    """The blob's body order, pinned by hand: for every layer, all K rows and then all V
    rows; within each, rows in token-major order (t, h).  A cache of 2 layers, 3 tokens,
    2 kv heads and head_dim 32 (one q8_0 block per row) is filled with a marker that names
    (layer, K/V, token, head, element), and every row is looked up at the offset
        32 + l*2*T*H*rb + which*T*H*rb + (t*H + h)*rb
    written out here rather than taken from the serializer.  Swapping K and V, t and h, or
    two layers moves some marker off its offset.  The form is the pages' layout-independent
    sequence state ("completion : allow the prompt to be processed under its own split
    mode", section "What this does"; "llama : switch the split mode of a live context",
    section "What this adds")."""
    L, T, H, hd = 2, 3, 2, 32
    rb = hd * 2 if kv == "f16" else 34
    cache = oracle.OracleCache(L, 8, H, hd, kv)

    def code(l, which, t, h):            # 0 .. 23, distinct for every row of the blob
        return ((l * 2 + which) * T + t) * H + h

    for l in range(L):
        for which in range(2):
            if kv == "f16":
                # row values code*32 + i: integers below 2048, exact in binary16
                rows = np.array([[[code(l, which, t, h) * 32 + i for i in range(hd)]
                                  for h in range(H)] for t in range(T)], dtype=np.float16)
            else:
                d16 = np.array([[[1.0 + code(l, which, t, h)] for h in range(H)]
                                for t in range(T)], dtype=np.float16)
                q = np.array([[[[(code(l, which, t, h) * 5 + i) % 251 - 125 for i in range(hd)]]
                               for h in range(H)] for t in range(T)], dtype=np.int8)
                rows = (d16, q)
            cache.set_stored(l, "kv"[which], rows, T)
    cache.n_past = T
    blob = oracle.state_bytes(cache, 1e6)
    assert len(blob) == 32 + L * 2 * T * H * rb
    for l in range(L):
        for which in range(2):
            for t in range(T):
                for h in range(H):
                    c = code(l, which, t, h)
                    off = 32 + l * 2 * T * H * rb + which * T * H * rb + (t * H + h) * rb
                    row = blob[off:off + rb]
                    if kv == "f16":
                        want = np.arange(c * 32, c * 32 + hd, dtype=np.float64).astype("<f2").tobytes()
                    else:
                        want = np.array([1.0 + c], dtype="<f2").tobytes() + bytes(
                            ((c * 5 + i) % 251 - 125) & 0xFF for i in range(hd))
                    assert row == want, (l, which, t, h)
    # the parser reads the same rows back from those offsets
    _, layers = oracle.parse_state(blob)
    for l in range(L):
        for which in range(2):
            got = layers[l][which]
            ref = cache.stored(l, "kv"[which], T)
            if kv == "f16":
                assert np.array_equal(got, ref)
            else:
                assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


@pytest.mark.parametrize("base", [TINY_DENSE, TINY_MOE])
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_f16_operand_mode_is_a_bounded_rounding_of_the_exact_mode(base, kv):
    """The "f16" operand mode takes every matrix-product operand as binary16: its weights
    are binary16 values, it differs from the exact mode by rounding-sized amounts (nonzero,
    well inside 1e-2), and its chunked and layer-major drivers agree."""
    w = base.with_(kv_type=kv)
    ql = q8_layers(w)
    x = synth.prompt_inputs(w)
    exact = oracle.OracleModel(w, ql).prefill_layer_major(x)
    m = oracle.OracleModel(w, ql, operands="f16")
    f16 = m.prefill_layer_major(x)
    e = rel(f16, exact)
    assert 1e-7 < e < 1e-2, e
    W = m.weights(0)
    for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        assert np.array_equal(oracle.to_f16(W[name]), W[name])
    assert rel(m.prefill(x, 7), f16) < 1e-3
