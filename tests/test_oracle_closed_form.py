"""Closed-form special cases of whole layer stacks: CPU pins of the oracle's end-to-end
hidden states.

With W_q = 0 every attention score is 0, and a softmax over equal scores is uniform: the
causal attention of query head h at token t is the plain mean of the cached V rows of kv
head h // G over positions 0..t (G query heads per kv head).  With W_down = 0 the FFN
adds exactly zero (all-zero q8_0 blocks decode to 0), dense or routed.  One layer is then

    x + concat_h( mean_{s <= t} V_{h // G}[s] ) W_o^T,
    V = f16(f32(rmsnorm(x) W_v^T))      (the f16 cache's stored form of V),

which the few lines of numpy below evaluate without the oracle's attention, RoPE, cache,
q8_0 decoder or drivers.  Two such layers pin the residual carried from layer to layer
and the order of the layers; chunk sizes of 1 and 3 tokens, the workload's own chunk
and the whole prompt pin the chunked driver, since the closed form does not depend on
the chunking.  A wrong GQA head map (h % Hkv), a dropped residual, a cache row written
at the wrong position or a chunk that does not see the rows before it each move the
result far outside the tolerance.
"""
import numpy as np
import pytest

import oracle
import synth
from model_inputs import TINY_DENSE, TINY_MOE, q8_layers


def decode_q8_0(b: np.ndarray, K: int) -> np.ndarray:
    """Interchange q8_0 rows [..., N][K/32 * 34] (per block: fp16 scale d, little
    endian, then 32 int8 codes q) -> float64 [..., N][K] with values d * q."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    nb = K // 32
    blk = b.reshape(b.shape[:-1] + (nb, 34))
    d = blk[..., :2].copy().view("<f2")[..., 0].astype(np.float64)
    q = blk[..., 2:].copy().view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(b.shape[:-1] + (K,))


def closed_form(w, layers, x: np.ndarray) -> np.ndarray:
    n, Hq, Hkv, hd = x.shape[0], w.n_head, w.n_kv_head, w.head_dim
    G = Hq // Hkv
    x = np.asarray(x, dtype=np.float64)
    for L in layers:
        y = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + w.rms_eps) * L["attn_norm"]
        Wv = decode_q8_0(L["wv"], w.d_model)
        Wo = decode_q8_0(L["wo"], Hq * hd)
        v = (y @ Wv.T).astype(np.float32).astype(np.float16).astype(np.float64)
        v = v.reshape(n, Hkv, hd)
        prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1, dtype=np.float64)[:, None, None]
        o = prefix_mean[:, np.arange(Hq) // G, :].reshape(n, Hq * hd)
        x = x + o @ Wo.T
    return x


def zero_q_and_down(layers):
    out = []
    for L in layers:
        L = dict(L)
        L["wq"] = np.zeros_like(L["wq"])
        L["w_down"] = np.zeros_like(L["w_down"])
        out.append(L)
    return out


@pytest.mark.parametrize("base", [TINY_DENSE, TINY_MOE])
def test_stack_with_zero_queries_and_zero_down_is_the_causal_prefix_mean(base):
    w = base.with_(kv_type="f16")
    layers = zero_q_and_down(q8_layers(w))
    m = oracle.OracleModel(w, layers)
    x = synth.prompt_inputs(w)
    ref = closed_form(w, layers, x)
    scale = float(np.max(np.abs(ref - x)))
    assert scale > 1e-3          # the attention terms are not negligible
    for chunk in (1, 3, w.chunk, w.n_prompt):
        got = m.prefill(x, chunk)
        assert float(np.max(np.abs(got - ref))) <= 1e-10 * scale, chunk
    got = m.prefill_layer_major(x)
    assert float(np.max(np.abs(got - ref))) <= 1e-10 * scale


def test_closed_form_rejects_a_transposed_head_map():
    """The pin has teeth: the same stack with the kv head of query head h taken as
    h % Hkv instead of h // G differs from the oracle by far more than the tolerance."""
    w = TINY_DENSE.with_(kv_type="f16")
    layers = zero_q_and_down(q8_layers(w))
    x = synth.prompt_inputs(w)
    got = oracle.OracleModel(w, layers).prefill(x, w.chunk)
    ref = closed_form(w, layers, x)
    Hq, Hkv, hd = w.n_head, w.n_kv_head, w.head_dim
    xx = np.asarray(x, dtype=np.float64)
    for L in layers:     # the same form with the wrong map
        y = xx / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + w.rms_eps) * L["attn_norm"]
        v = (y @ decode_q8_0(L["wv"], w.d_model).T).astype(np.float32).astype(np.float16)
        v = v.astype(np.float64).reshape(-1, Hkv, hd)
        pm = np.cumsum(v, axis=0) / np.arange(1, v.shape[0] + 1)[:, None, None]
        o = pm[:, np.arange(Hq) % Hkv, :].reshape(v.shape[0], Hq * hd)
        xx = xx + o @ decode_q8_0(L["wo"], Hq * hd).T
    scale = float(np.max(np.abs(ref - x)))
    assert float(np.max(np.abs(got - ref))) <= 1e-10 * scale
    assert float(np.max(np.abs(got - xx))) > 1e-3 * scale
