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
