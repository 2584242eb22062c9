"""Pins for the cost fit, the pipeline chunk rule and the input generator (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_linear_fit_recovers_known_cost_exactly():
    C = np.array([128, 256, 384, 512, 1024, 2048, 4096, 8192], dtype=np.float64)
    b, a = 80.0, 0.08
    fb, fa, r2 = oracle.fit_linear(C, b + a * C)
    assert abs(fb - b) < 1e-9 and abs(fa - a) < 1e-12 and r2 == pytest.approx(1.0)
    # two chunk sizes: the fit is the line through the two points
    fb, fa, _ = oracle.fit_linear([512, 2048], [b + a * 512, b + a * 2048])
    assert fb == pytest.approx(b) and fa == pytest.approx(a)
    qb, qa, qc = oracle.fit_quadratic(C, 3.0 + 0.5 * C + 1e-4 * C * C)
    assert (qb, qa, qc) == pytest.approx((3.0, 0.5, 1e-4), rel=1e-6)


def load_chunk_table():
    rows = []
    with open(os.path.join(GOLDEN, "pipeline_chunks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                n, stages, chunk = (int(v) for v in line.split())
                rows.append((n, stages, chunk))
    return rows


def test_pipeline_chunk_reproduces_page_table():
    rows = load_chunk_table()
    assert len(rows) == 4
    for n, stages, chunk in rows:
        assert oracle.pipeline_chunk(n, 8192, stages) == chunk
        assert oracle.pipeline_chunk(n, 8192, stages, b_over_a=1000.0) == chunk


def test_pipeline_chunk_limits():
    assert oracle.pipeline_chunk(300, 8192, 4) == 300            # one chunk: today's path
    assert oracle.pipeline_chunk(10041, 8192, 1) == 8192         # one stage: largest chunk
    assert oracle.pipeline_chunk(100000, 2048, 4) == 2048        # capped by the buffers
    assert oracle.pipeline_chunk(10041, 8192, 2) == 2560         # two stages, evened out


def test_synth_numpy_and_torch_paths_are_bit_identical():
    torch = pytest.importorskip("torch")
    for seed, shape in [(1, (1000,)), (123456789, (37, 51))]:
        a = synth.normal(seed, shape)
        b = synth.normal_torch(seed, shape).numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    x = synth.normal(5, (1 << 18,), scale=1.0).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.array_equal(synth.normal(5, (10,)), synth.normal(5, (10,)))
    assert not np.array_equal(synth.normal(5, (10,)), synth.normal(6, (10,)))


def test_last_logits_by_hand():
    """Two head rows of 32 values each: row 0 holds 127 in column 3 and zeros elsewhere, so
    its block scale is exactly 1 and its logit is y_3 * 127; row 1 holds -2 in column 0 and 2
    in column 31 (scale 2/127 after fp16 rounding).  x is constant, so RMSNorm gives 1 * gamma."""
    d = 32
    W = np.zeros((2, d), np.float32)
    W[0, 3] = 127.0
    W[1, 0], W[1, 31] = -2.0, 2.0
    head = oracle.q8_0_encode_bytes(W)
    gamma = np.arange(1, d + 1, dtype=np.float32) / 16.0
    x = np.full(d, 0.5, np.float32)
    got = oracle.last_logits(x, gamma, head, d, 1e-6)
    y = 0.5 / np.sqrt(0.25 + 1e-6) * gamma.astype(np.float64)
    s1 = float(np.float16(np.float32(2.0) / np.float32(127.0)))   # stored scale of row 1
    assert abs(got[0] - 127.0 * y[3]) < 1e-12
    assert abs(got[1] - s1 * 127.0 * (y[31] - y[0])) < 1e-12


def test_last_logits_chunk_invariant():
    """The last-position logits of a chunked prefill equal those of the whole prompt at once."""
    from model_inputs import TINY_DENSE, q8_layers
    w = TINY_DENSE
    m = oracle.OracleModel(w, q8_layers(w))
    x = synth.prompt_inputs(w)
    head = oracle.q8_0_encode_bytes(synth.normal(synth.tensor_seed("head", 97, w.d_model), (97, w.d_model)))
    gamma = np.ones(w.d_model, np.float32)
    full = oracle.last_logits(m.prefill_layer_major(x)[-1], gamma, head, w.d_model, 1e-6)
    chunked = oracle.last_logits(m.prefill(x, 3)[-1], gamma, head, w.d_model, 1e-6)
    assert np.max(np.abs(full - chunked)) <= 1e-12 * np.max(np.abs(full))
